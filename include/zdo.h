/*
 * zdo.h — one data-parallel rank's share of a distributed-optimizer step
 * (ZeRO-1 style, as in Megatron-LM's DistributedOptimizer) on AMD Instinct
 * MI355X (gfx950).
 *
 * The method (page "04 · 分布式优化器", a Megatron-LM code-reading chapter):
 * the grads of one dtype live in one flat 1-D buffer cut into buckets (§2);
 * each bucket is padded to a multiple of the DP size D (§5) and split into D
 * equal contiguous ranges, rank r owning range r whatever parameters it cuts
 * (§2, §3); the grads are scaled (§5), reduce-scattered so each rank keeps
 * the sum over its range (§4.2), copied into the rank's fp32 main-grad
 * shard through the four-way range map (§4.1, §4.3), Adam runs on the fp32
 * master/m/v shard only (§4.3), and the updated parameters are written back
 * as bf16 into the owned range of the parameter buffer (§4.3); the
 * all-gather of the parameter buffers then gives every rank the whole
 * updated parameters (§4.4, all_gather_params). force_all_reduce produces
 * the whole reduced buffer instead of the reduce-scatter (§5).
 *
 * On one GPU, the D ranks' contributions are D replica buffers in this
 * GPU's memory; the library sums them itself (no collective library).
 *
 * Conventions for every call:
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Device pointers are caller-owned, must be 16-byte aligned (device
 *     scalars: naturally aligned), and point to memory of the device the
 *     plan was built on. Host arrays (the replica pointer list, param_numel,
 *     hp) are read during the call only.
 *   - `stream` is a hipStream_t passed as void * (NULL = the default
 *     stream), so that this header needs no HIP header; a hipStream_t
 *     converts to it implicitly. Calls that take one only enqueue work on it
 *     and return; they never allocate device memory and never synchronise
 *     the host.
 *   - A launch captured into a HIP graph replays with the arguments of its
 *     capture. For the Adam calls these include the bias corrections of
 *     hp->step, formed on the host at the call: a captured step is valid
 *     for that one t, and a graph that replays several steps needs one
 *     capture per t.
 *   - Coordinates of a buffer: ZDO_WORLD indexes the whole padded buffer
 *     [0, N); ZDO_LOCAL indexes the rank's shard [0, L).
 *   - The contributions a call sums (n_replicas / n_grads, 1..ZDO_MAX_REPLICAS,
 *     each a device pointer in a host array) are summed in the order given.
 *     The plain step passes the D ranks' contributions. With several
 *     distributed-optimizer instances (page 1, §5: the reduce-scatter runs
 *     within each instance of D ranks, then an all-reduce across the
 *     instances), call reduce_scatter_local once per instance on its D
 *     contributions, then pass the instances' results, in instance order and
 *     with scale 1, as the contributions of sharded_adam_step (or of
 *     reduce_scatter_local for the reduced gradient alone); one contribution
 *     with scale 1 is an already reduced gradient, taken as it is.
 *   - Every call returns ZDO_OK (0) or a negative ZDO_E* code; the message of
 *     the last failing call on this thread is zdo_last_error(). No call
 *     aborts or throws. Faults inside a kernel surface when the caller
 *     synchronises the stream.
 *
 * Arithmetic (fixed, so results are reproducible bit for bit):
 *   per owned element w:  s_j = bf16(fp32(g_j[w]) * scale), j = 0..n-1
 *                         acc = s_0 + s_1 + ... + s_{n-1}   (fp32, this order)
 *                         g   = fp32(bf16(acc))
 *   Adam (Kingma & Ba, Algorithm 1, with weight decay decoupled and scaled by
 *   lr as in Loshchilov & Hutter), each step one fp32 IEEE operation, no FMA:
 *     m' = b1*m + (1-b1)*g        v' = b2*v + (1-b2)*(g*g)
 *     p' = p - lr*( (m'/bc1) / (sqrt(v'/bc2) + eps) + wd*p )
 *   with 1-b1, 1-b2 in fp32 and bc_i = 1 - b_i^t computed in double by t
 *   products and rounded once. bf16() is round-to-nearest-even, overflow to
 *   Inf, subnormals kept, NaN stays NaN.
 */
#ifndef ZDO_H
#define ZDO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZDO_OK 0
#define ZDO_EINVAL (-1)   /* bad argument (size, rank, coords, count, NULL) */
#define ZDO_EALIGN (-2)   /* a device pointer is not aligned as required */
#define ZDO_EALIAS (-3)   /* outputs overlap each other or the inputs illegally */
#define ZDO_EHIP (-4)     /* HIP runtime or launch failure; no device for the plan */
#define ZDO_ENOMEM (-5)   /* host or device allocation failed */

#define ZDO_WORLD 0
#define ZDO_LOCAL 1

#define ZDO_MAX_REPLICAS 64   /* largest D (and replica count) a launch accepts */

typedef struct zdo_plan zdo_plan;

/* Half-open [start, end) of element indices (page 1, §4.1 "Range"). */
typedef struct {
    int64_t start, end;
} zdo_range;

/* One parameter's piece inside the rank's range of one bucket (page 1,
 * §4.1): the same elements described four ways, all translations of one
 * another. shard_offset is where gbuf_world.start sits in the rank's fp32
 * shard (master/m/v/main grad, LOCAL coordinates). 80 bytes, no padding. */
typedef struct {
    int32_t param_index, bucket_index;
    zdo_range gbuf_world;            /* in the whole buffer */
    zdo_range gbuf_world_in_bucket;  /* relative to the bucket start */
    zdo_range gbuf_local;            /* relative to the rank's range start */
    zdo_range param;                 /* inside the parameter itself */
    int64_t shard_offset;
} zdo_piece;

/* One bucket. shard_numel = padded_numel / D; the rank's range of the bucket
 * is [offset + rank*shard_numel, +shard_numel) in WORLD coordinates and
 * [shard_base, shard_base + shard_numel) in LOCAL coordinates. */
typedef struct {
    int64_t offset, numel, padded_numel, shard_numel, shard_base;
} zdo_bucket;

/* Adam hyper-parameters for one step; step is t >= 1. */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    int32_t reserved;   /* must be 0 */
    int64_t step;
} zdo_adam;

/* ---- plan: layout and range map (host) ----------------------------------- */

/* Lays out n_params parameters of the given element counts (each >= 1) in
 * order in one flat buffer; cuts buckets greedily (a bucket closes right after
 * the parameter that brings it to >= bucket_numel elements, or after the last
 * parameter; a parameter never spans two buckets); pads each bucket at its
 * tail to a multiple of dp_size; and builds rank `rank`'s range map (page 1,
 * §2, §3, §4.1, §5). The rank's fp32 shard places each bucket's local view at
 * the first slot >= the previous view's end that is congruent to the range's
 * WORLD start modulo 64, so every LOCAL index is congruent to its WORLD index
 * modulo 64 (gap slots, < 64 per bucket, and padding slots are never
 * touched). With buffers aligned to 128 bytes, every stream then crosses
 * cache lines at the same elements, which the kernels' tiles follow.
 * If a HIP device is present, the plan's segment table is uploaded to the
 * current device (the plan's device); otherwise the plan is host-only and
 * the launch calls fail with ZDO_EHIP. *out receives the plan, owned by the
 * caller until zdo_plan_destroy. Errors: ZDO_EINVAL (n_params < 1, a size
 * < 1, bucket_numel < 1, dp_size < 1 or > ZDO_MAX_REPLICAS, rank outside
 * [0, dp_size), NULL), ZDO_ENOMEM, ZDO_EHIP (upload failed). */
int build_range_map(const int64_t *param_numel, int32_t n_params, int64_t bucket_numel,
                    int32_t dp_size, int32_t rank, zdo_plan **out);

void zdo_plan_destroy(zdo_plan *plan);

int64_t zdo_plan_buffer_numel(const zdo_plan *plan);  /* N: padded buffer length */
int64_t zdo_plan_shard_numel(const zdo_plan *plan);   /* L: shard length, gaps and padding included */
int64_t zdo_plan_owned_numel(const zdo_plan *plan);   /* E: parameter elements the rank owns */
int32_t zdo_plan_dp_size(const zdo_plan *plan);
int32_t zdo_plan_rank(const zdo_plan *plan);

/* Two-call queries: with out == NULL (or cap too small) only *n is set. */
int zdo_plan_buckets(const zdo_plan *plan, zdo_bucket *out, int32_t cap, int32_t *n);
int zdo_plan_pieces(const zdo_plan *plan, zdo_piece *out, int64_t cap, int64_t *n);

/* The same five plan calls under the short names of the range-map interface
 * (page 1, §4.1: the map builders and their Range tables). Each is the
 * zdo_-prefixed call above, with the same arguments, results and errors. */
int plan_buckets(const zdo_plan *plan, zdo_bucket *out, int32_t cap, int32_t *n);
int plan_pieces(const zdo_plan *plan, zdo_piece *out, int64_t cap, int64_t *n);
int64_t plan_buffer_numel(const zdo_plan *plan);
int64_t plan_shard_numel(const zdo_plan *plan);
void plan_destroy(zdo_plan *plan);

/* ---- device work ---------------------------------------------------------- */

/* Reduce-scatter of the D contributions over the rank's whole range of every
 * bucket, padding included (page 1, §4.2, with the scaling of §5 first).
 * replicas: host array of n_replicas device pointers (the D ranks'
 * contributions, or see the instances rule above), each a bf16 buffer of N
 * (replica_coords = ZDO_WORLD) or L (ZDO_LOCAL) elements.
 * out: bf16, N elements (out_coords = ZDO_WORLD) or L (ZDO_LOCAL); only the
 * rank's ranges are written. out may coincide exactly with one replica when
 * both use the same coordinates (in place, like a reduce-scatter into the
 * grad buffer's own local view); any other overlap is ZDO_EALIAS. */
int reduce_scatter_local(const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas,
                         int32_t replica_coords, float scale, uint16_t *out, int32_t out_coords,
                         void *stream);

/* All-reduce of the D contributions over the whole padded buffer (page 1, §5,
 * force_all_reduce: the full reduced grads instead of the rank's share).
 * Same arithmetic as reduce_scatter_local; independent of the rank.
 * replicas: n_replicas device bf16 buffers of N elements. out_full:
 * bf16, N elements; it may coincide exactly with one replica. */
int force_all_reduce(const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas,
                     float scale, uint16_t *out_full, void *stream);

/* The rank's optimizer step, fused: reduce the n_grads contributions over
 * every owned parameter element, copy into the fp32 main grad through the
 * range map, Adam on master/exp_avg/exp_avg_sq, and write bf16(master') into
 * param_out (page 1, §4.2, §4.3, §5). Padding and elements of other ranks
 * are neither read from the state nor written anywhere.
 * grads: host array of n_grads device pointers: the D replicas, or 1 already
 * reduced buffer (e.g. the output of reduce_scatter_local or
 * force_all_reduce, with scale 1 to leave it unchanged), or the instances'
 * reduce-scatter results (see above); bf16 of N (grad_coords ZDO_WORLD) or
 * L (ZDO_LOCAL) elements.
 * master, exp_avg, exp_avg_sq: fp32, L elements each (LOCAL), updated in
 * place; pairwise disjoint. param_out: bf16, N (param_coords ZDO_WORLD) or L
 * (ZDO_LOCAL) elements, or NULL to skip the write-back. main_grad_out: fp32,
 * L elements, or NULL; receives the fp32 main grad (a debugging output).
 * hp: host pointer; hp->step >= 1. Outputs must not overlap each other or
 * the grads (ZDO_EALIAS). */
int sharded_adam_step(const zdo_plan *plan, const uint16_t *const *grads, int32_t n_grads,
                      int32_t grad_coords, float scale, float *master, float *exp_avg,
                      float *exp_avg_sq, uint16_t *param_out, int32_t param_coords,
                      const zdo_adam *hp, float *main_grad_out, void *stream);

/* sharded_adam_step for n_instances distributed-optimizer instances of D
 * ranks each, in one pass (page 1, §5: the reduce-scatter runs within each
 * instance, then an all-reduce across the instances). grads: host array of
 * n_instances * D device pointers, instance-major (instance i's D
 * contributions, in rank order, at [i*D, i*D + D)), all in grad_coords.
 * Each instance's contributions are summed as sharded_adam_step sums them
 * (scale applied to each term first) and rounded to bf16; those n_instances
 * bf16 sums are added in fp32 in instance order and rounded to bf16, and the
 * step continues as sharded_adam_step. The result equals reduce_scatter_local
 * per instance followed by sharded_adam_step on the instance results with
 * scale 1, bit for bit, without the intermediate buffers. 1 <= n_instances,
 * n_instances * D <= ZDO_MAX_REPLICAS (else ZDO_EINVAL). Other arguments and
 * rules as sharded_adam_step. */
int sharded_adam_step_instances(const zdo_plan *plan, const uint16_t *const *grads, int32_t n_instances,
                                int32_t grad_coords, float scale, float *master, float *exp_avg,
                                float *exp_avg_sq, uint16_t *param_out, int32_t param_coords,
                                const zdo_adam *hp, float *main_grad_out, void *stream);

/* bf16(master) into the owned parameter elements of param_out (page 1, §4.3:
 * the updated master shard copied back into the buffer's owned range).
 * master: fp32, L elements; param_out: bf16, N (ZDO_WORLD) or L (ZDO_LOCAL)
 * elements; must not overlap. */
int writeback_params(const zdo_plan *plan, const float *master, uint16_t *param_out,
                     int32_t param_coords, void *stream);

/* Page 1, §4.4: after the step, every bucket's parameter buffer is
 * all-gathered, so that every rank holds the whole updated parameters (the
 * ZeRO-1 loop: reduce-scatter of the grads, sharded step, all-gather of the
 * parameters). This is one rank's side of it: rank j's range of every padded
 * bucket (padding included, as the collective over equal ranges moves it) is
 * copied from params[j] into out. params: host array of n_params (== D)
 * device pointers, bf16 parameter buffers of N elements in WORLD
 * coordinates, params[j] holding rank j's write-back (e.g. sharded_adam_step
 * or writeback_params with param_coords ZDO_WORLD). out: bf16, N elements;
 * it may coincide exactly with one or more params[j] (in place, typically
 * the plan's own rank: those ranges are already there and are not copied)
 * and must not otherwise overlap any of them (ZDO_EALIAS). The plan may be
 * any rank's: the bucket layout is the same for all. n_params != D:
 * ZDO_EINVAL. */
int all_gather_params(const zdo_plan *plan, const uint16_t *const *params, int32_t n_params,
                      uint16_t *out, void *stream);

/* ---- bucket by bucket ---------------------------------------------------------
 * Page 1, §2 and §4.2: a bucket's collective starts as soon as the grads of
 * its bucket are ready, bucket by bucket during the backward pass. These two
 * calls do reduce_scatter_local's and sharded_adam_step's work for the
 * buckets [bucket_begin, bucket_end) only (0 <= begin <= end <= number of
 * buckets; an empty range does nothing). Calls over disjoint ranges that
 * together cover every bucket, in any order, give the full call's results bit
 * for bit. Other arguments and rules as the full calls. */
int reduce_scatter_local_buckets(const zdo_plan *plan, int32_t bucket_begin, int32_t bucket_end,
                                 const uint16_t *const *replicas, int32_t n_replicas, int32_t replica_coords,
                                 float scale, uint16_t *out, int32_t out_coords, void *stream);
int sharded_adam_step_buckets(const zdo_plan *plan, int32_t bucket_begin, int32_t bucket_end,
                              const uint16_t *const *grads, int32_t n_grads, int32_t grad_coords, float scale,
                              float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param_out,
                              int32_t param_coords, const zdo_adam *hp, float *main_grad_out, void *stream);

/* The same two calls for several bucket ranges at once, in one launch (page
 * 1, §4.2: the buckets of a group are handled together, their communication
 * coalesced into one kernel). bucket_ranges: host array of n_ranges
 * (begin, end) pairs, each with 0 <= begin <= end <= number of buckets,
 * pairwise disjoint (overlap: ZDO_EINVAL), in any order; empty ranges are
 * skipped and ranges that touch are merged. One launch covers up to 16
 * disjoint runs of tiles; longer lists take one launch per 16 runs. The
 * results equal the per-range calls bit for bit. n_ranges = 0 does
 * nothing. Other arguments and rules as the full calls. */
int reduce_scatter_local_bucket_list(const zdo_plan *plan, const int32_t *bucket_ranges, int32_t n_ranges,
                                     const uint16_t *const *replicas, int32_t n_replicas, int32_t replica_coords,
                                     float scale, uint16_t *out, int32_t out_coords, void *stream);
int sharded_adam_step_bucket_list(const zdo_plan *plan, const int32_t *bucket_ranges, int32_t n_ranges,
                                  const uint16_t *const *grads, int32_t n_grads, int32_t grad_coords, float scale,
                                  float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param_out,
                                  int32_t param_coords, const zdo_adam *hp, float *main_grad_out, void *stream);

/* ---- global-norm clipping ---------------------------------------------------
 * The distributed-training notes, §8.3: each rank's squared gradient sum is
 * all-reduced into the global norm sqrt(sum_i ||g_i||^2), and the gradients
 * are clipped before the optimizer update. Here: g is the rank's reduced
 * bf16 gradient over its owned parameter elements (as sharded_adam_step
 * computes it); grad_norm_sq gives the rank's share, the caller sums the
 * ranks' shares (a collective across GPUs; a device array here) with
 * clip_coefficient, and sharded_adam_step_clipped applies the coefficient.
 * Nothing here synchronises the host: the coefficient stays in device memory.
 */

/* Workspace bytes grad_norm_sq needs for this plan: 8 per 512-element tile of
 * the rank's owned elements plus 8 KiB. */
int64_t zdo_plan_norm_workspace_bytes(const zdo_plan *plan);

/* The rank's squared gradient norm: sum over its owned parameter elements of
 * g^2, g = bf16(sum_j bf16(scale * g_j)) exactly as in sharded_adam_step,
 * squares (exact in fp64) summed in fp64 in a fixed order: per 512-element
 * tile (lanes' 8 elements in order, then a fixed butterfly over the 64
 * lanes) into `workspace`, then the tile sums in two fixed levels (at most
 * 1024 contiguous runs, then the runs) into *norm_sq_out. The order
 * depends only on the plan, so the result is bit-identical run to run;
 * against a sequential fp64 sum it differs only by fp64 rounding.
 * replicas / n_replicas / replica_coords: as sharded_adam_step's grads.
 * reduced_out: NULL, or bf16 N (out_coords ZDO_WORLD) / L (ZDO_LOCAL)
 * elements receiving g at the owned elements only (then sharded_adam_step
 * with n_grads = 1 and scale 1 on it reads 2 bytes per element instead of
 * 2D); it may coincide exactly with a replica in the same coordinates.
 * workspace: device, zdo_plan_norm_workspace_bytes(plan) bytes, 16-byte
 * aligned, used by this call only until it completes on `stream` (calls that
 * overlap in time need separate workspaces). norm_sq_out: device double,
 * 8-byte aligned. A rank that owns nothing gets 0. */
int grad_norm_sq(const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas,
                 int32_t replica_coords, float scale, uint16_t *reduced_out, int32_t out_coords,
                 void *workspace, double *norm_sq_out, void *stream);

/* grad_norm_sq without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The per-tile partials go to a static
 * device array of the library, ZDO_NO_ALLOC_SCRATCH_BYTES bytes on each GPU
 * it runs on (held until the process ends); the call itself allocates
 * nothing. Same kernels, same fixed summation order, so the results equal
 * grad_norm_sq's bit for bit. The plan's zdo_plan_norm_workspace_bytes must
 * not exceed ZDO_NO_ALLOC_SCRATCH_BYTES (64 MiB: up to 8,387,584 tiles of 512
 * owned elements, about 4.29e9 elements per rank), else ZDO_EINVAL before
 * anything is enqueued. Every call on one GPU uses that GPU's one array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and give wrong results; calls ordered on one stream are safe. Other
 * arguments and rules as grad_norm_sq. */
#define ZDO_NO_ALLOC_SCRATCH_BYTES (64u << 20)
int grad_norm_sq_no_alloc(const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas,
                          int32_t replica_coords, float scale, uint16_t *reduced_out, int32_t out_coords,
                          double *norm_sq_out, void *stream);

/* From n_parts squared norms (device doubles, e.g. every rank's grad_norm_sq),
 * summed in index order in fp64: norm = sqrt(total) and the clipping
 * coefficient min(1, max_norm / (norm + 1e-6)) computed in fp64 and rounded to
 * fp32, written to *coeff_out (device float, 4-byte aligned); NaN if the norm
 * is not finite (found-inf: sharded_adam_step_clipped then skips the step).
 * norm_out: NULL or a device double receiving the norm. One work-item. */
int clip_coefficient(const double *norm_sq_parts, int32_t n_parts, float max_norm, float *coeff_out,
                     double *norm_out, void *stream);

/* sharded_adam_step with global-norm clipping: the fp32 main grad is
 * multiplied by *grad_coeff (a device float read by the kernel, e.g. from
 * clip_coefficient) before Adam, and main_grad_out receives the product. If
 * *grad_coeff is NaN the call changes nothing (found-inf skip). With
 * *grad_coeff == 1 the results equal sharded_adam_step's bit for bit. All
 * other arguments and rules as sharded_adam_step. */
int sharded_adam_step_clipped(const zdo_plan *plan, const uint16_t *const *grads, int32_t n_grads,
                              int32_t grad_coords, float scale, float *master, float *exp_avg,
                              float *exp_avg_sq, uint16_t *param_out, int32_t param_coords,
                              const zdo_adam *hp, const float *grad_coeff, float *main_grad_out,
                              void *stream);

/* ---- measurement helper (not part of the method) -------------------------- */

/* Plain device copy of `bytes` bytes (a multiple of 16) from src to dst,
 * non-overlapping, both 16-byte aligned: the streaming-bandwidth and
 * counter-calibration reference for the kernels above. */
int zdo_device_copy(void *dst, const void *src, int64_t bytes, void *stream);

/* Which stores zdo_stream_probe makes. */
#define ZDO_PROBE_STORE_ALL 0   /* the step's: state rewritten, out written */
#define ZDO_PROBE_STORE_OUT 1   /* out written, the state only read */
#define ZDO_PROBE_STORE_NONE 2  /* loads only: one 4-byte word per tile into out */

/* The fused step's memory traffic with trivial arithmetic: the ceiling of its
 * stream shape, measured beside the step (a measurement reference, not part
 * of the method). Over n elements (a multiple of 512, >= 0), in tiles of 512
 * in the step's tile and lane layout, every access non-temporal: each of the
 * n_reads bf16 buffers reads[j] is read once (n_reads = 8, 16 or 32) and the
 * three fp32 buffers state0..2 are read. Lane l of a tile holds the 16-byte
 * chunk [8l, 8l + 8) of each read buffer and the quads [4l, 4l + 4) and
 * [256 + 4l, 256 + 4l + 4) of each state buffer; x is the XOR of its read
 * chunks (four 32-bit words). What is then stored, by `stores`:
 *   ZDO_PROBE_STORE_ALL (2*n_reads + 26 bytes per element, the step's count):
 *     every state value gains the exponent bits of x[0]^x[1]^x[2]^x[3], and
 *     quad h of out gets the old master[0] and exp_avg[1] bits of quad h,
 *     XORed with x[2h] and x[2h+1];
 *   ZDO_PROBE_STORE_OUT (2*n_reads + 14): the state is not stored; quad h of
 *     out gets x[2h] ^ S_h and x[2h+1] ^ S_h, S_h the XOR of the 12 state
 *     words of quad h;
 *   ZDO_PROBE_STORE_NONE (2*n_reads + 12): nothing but, per tile t, the
 *     32-bit word at out[2t, 2t+2) = the XOR over the tile's 64 lanes of
 *     x[0]^x[1]^x[2]^x[3]^S_0^S_1; the rest of out is left as it was.
 * waves_per_cu caps the workgroups per compute unit (0: no cap). All buffers
 * device, 16-byte aligned, n elements, pairwise disjoint (ZDO_EALIAS); the
 * current device's LDS size sets the cap. */
int zdo_stream_probe(const uint16_t *const *reads, int32_t n_reads, float *state0, float *state1, float *state2,
                     uint16_t *out, int64_t n, int32_t stores, int32_t waves_per_cu, void *stream);

const char *zdo_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZDO_H */
