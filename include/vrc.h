/*
 * vrc.h -- virtual-rank collectives on one AMD Instinct MI355X (gfx950).
 *
 * N "virtual ranks" are N equally sized buffers that all live in the HBM of
 * the one GPU the calls run on.  The library runs the ring all-reduce and
 * its reduce-scatter and all-gather halves over them with hand-written HIP
 * kernels.  Two kernel families are offered:
 *
 *   VRC_RING  - step-faithful ring: one chunk-add launch per reduce-scatter
 *               step and one chunk-copy launch per all-gather step, in the
 *               chunk order of the ring schedule below;
 *   VRC_FUSED - one launch that reads every input once, accumulates in fp32
 *               (uint32 for int32) and writes every output once (the naive
 *               "one collector sums and hands the result back" all-reduce).
 *
 * Sources (pages are named by address; sections by their heading):
 *   [RS]    ai6s.net/6a102b5410ee7a33f2746c06.html, "hcomm 与 HCCL 的关系":
 *           AllReduce = ReduceScatter + AllGather; the simplified
 *           ReduceScatter listing (send/recv one chunk per step, add the
 *           received chunk, move both chunk indices down by one).
 *   [RING]  hwcomputing.csdn.net/6a0dc11a10ee7a33f273f7fd.html, "Ring
 *           通信为什么常见": logical ring 0->1->..->N-1->0, N blocks, N-1
 *           reduce-scatter steps and N-1 all-gather steps, traffic
 *           2(N-1)*S/N per rank.
 *   [NAIVE] same page, "为什么大模型训练离不开通信": the collector all-reduce.
 *   [REM]   ai6s.net/6a157e6510ee7a33f27553e9.html, "自定义通信模式": equal
 *           chunks, the last chunk takes the remainder.
 *   [TP]    ai6s.net/6a0dd5b5662f9a54cb75ef90.html, "TP 通信": all-reduce of
 *           activations and all-gather along a dimension.
 *   [INFER] ai6s.net/6a102b5410ee7a33f2746c06.html, "分布式推理中的通信" and
 *           "hcomm 在推理场景中的使用": all-gather of attention-head slices;
 *           AllGather(send_buf, recv_buf, count, comm).
 *   [OVERLAP] www.bjdmk.com.cn/news/5966809/, section 4 (compute/comm
 *           overlap): collectives are enqueued on a stream.
 *   [TREE]  ai6s.net/6a102b5410ee7a33f2746c06.html, "分布式推理中的通信":
 *           the all-gather has a ring form and a tree form, chosen by data
 *           size (the tree itself is not defined there).
 *
 * Chunking.  A buffer of `count` elements has chunks c = 0..N-1: with
 * base = count / N, chunk c is [c*base, (c+1)*base) for c < N-1 and the last
 * chunk is [(N-1)*base, count) [REM].  Chunks are empty when count < N.
 *
 * Ring schedule [RS][RING].  Reduce-scatter step s = 0..N-2: rank r adds
 * the partial of chunk (r-1-s) held by rank r-1 into its own copy.  After
 * step N-2 rank r holds the complete chunk r+1.  All-gather step s: rank r
 * copies chunk (r-s) from rank r-1.  Every chunk c is therefore summed as
 * ((x_c + x_{c+1}) + x_{c+2}) + ... + x_{c+N-1} (indices mod N), each
 * partial rounded to the storage type.
 *
 * Arithmetic.  int32: two's-complement wrap.  fp32: IEEE add, round to
 * nearest even, no FMA, denormals kept.  fp16/bf16: widen exactly to fp32,
 * add in fp32, round to nearest even into the storage type (ring mode
 * rounds every partial; fused mode rounds once after the rank-order fold
 * x_0 + x_1 + ... + x_{N-1}).
 *
 * Conventions shared by all calls.
 *   send, recv  Host arrays of `nranks` DEVICE pointers (rank r's input and
 *               output).  The arrays are read during the call only; the
 *               buffers stay owned by the caller.  The library allocates no
 *               memory and keeps no pointer after returning; its only
 *               device state is an 8-byte count per element type in its own
 *               device memory (see Threads).
 *   count       Elements per rank INPUT buffer, at most 2^56 (larger values,
 *               whose byte sizes could wrap, return VRC_ERR_INVALID_ARG).
 *   stream      A hipStream_t (NULL = the null stream) on the current device.
 *               Work is enqueued asynchronously; the call returns before it
 *               finishes.  Errors raised by running kernels surface at the
 *               caller's next synchronisation, not here.
 *   Alignment   Any element-aligned pointer works, and every operand moves
 *               in 16-byte vectors whatever its offset.  A region's vectors
 *               start where its destination crosses a 128-byte boundary (the
 *               elements before it and the last partial vector run scalar).
 *               Where the outputs of a single-launch all-reduce sit on
 *               different offsets modulo 128 bytes, VRC_FUSED, VRC_HD_ORDER
 *               and VRC_RING_ORDER store each output on its own 128-byte
 *               grid (unless an output is its own input).  Operands on other
 *               offsets cost some bandwidth: about 5-10 % for the all-reduce
 *               with every input and output on its own offset; about 45 %
 *               for VRC_RING_CHAINED, whose partials keep the reference grid.
 *   Errors      Argument errors return before anything is enqueued.  After
 *               each launch the library reads (and so clears) the calling
 *               thread's last HIP error: a failed launch returns VRC_ERR_HIP
 *               with its code in vrc_last_hip_error(), and so does an error
 *               that an earlier HIP call left pending on the thread.
 *   Threads     Calls are re-entrant and thread-safe; calls that overlap on
 *               the same buffers race like any two kernels would.  Phased
 *               all-reduces (below) that run at the same time on one GPU
 *               share their workgroups' meeting count: each still finishes
 *               with its own exact result, but their phases may fall out of
 *               step (every wait is bounded by the workgroup's own read
 *               time).
 *   Runtime     The library calls the HIP runtime (libamdhip64.so.7) that is
 *               already loaded in the process.  A process that also uses
 *               PyTorch-ROCm, which bundles its own copy, must load PyTorch
 *               before this library so that both use one runtime.
 */
#ifndef VRC_H
#define VRC_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VRC_VERSION 106 /* 1.0.6: phased fused, butterfly and ring-order all-reduce launches in vrc_plan */
#define VRC_MAX_RANKS 16

struct ihipStream_t;
typedef struct ihipStream_t* vrc_stream_t; /* the same type as hipStream_t */
struct ihipEvent_t;
typedef struct ihipEvent_t* vrc_event_t;   /* the same type as hipEvent_t */

typedef enum { VRC_INT32 = 0, VRC_FP32 = 1, VRC_FP16 = 2, VRC_BF16 = 3 } vrc_dtype_t;
typedef enum { VRC_SUM = 0 } vrc_op_t;
/* Kernel family.  VRC_RING, VRC_RING_CHAINED and VRC_RING_ORDER return the same
 * bits (the ring's summation order, every partial rounded to the storage
 * type); VRC_FUSED folds in rank order in fp32 and rounds once.
 *   VRC_RING          one launch per ring step: 2(N-1) launches for the
 *                     all-reduce, N-1 for either half.
 *   VRC_FUSED         one launch; every input read once, every output
 *                     written once.  From 6 ranks, with every output on
 *                     one 128-byte grid and at least three phases of work,
 *                     the launch runs in phases: one 256-lane workgroup per
 *                     CU folds 0.5-1 GiB of the inputs, the grid meets, and
 *                     the sums are written (reads then do not wait behind
 *                     writes; about 5-9 % faster on MI355X).  The meeting
 *                     only shapes timing: results are the same bits.
 *   VRC_RING_CHAINED  one launch issuing the per-step reads and writes of
 *                     VRC_RING: each element of chunk c walks its chunk's
 *                     ring steps through the rank buffers (every element's
 *                     steps depend only on that element, so no grid-wide
 *                     barrier is needed).  A partial is read back right
 *                     after it is stored, so the cache serves most of those
 *                     reads.
 *   VRC_RING_ORDER    one launch with the fused traffic (read N, write N):
 *                     the ring's partials stay in registers, in phases from
 *                     6 ranks as VRC_FUSED.  For the all-gather it equals
 *                     VRC_FUSED.
 * Halving-doubling [TP] (nranks must be a power of two, else
 * VRC_ERR_INVALID_ARG): recursive halving reduce-scatter with distances N/2,
 * N/4, ..., 1 (rank r pairs with r XOR d, keeps the half of its block range
 * that holds block r and adds the partner's copy of it), then recursive
 * doubling all-gather with distances 1, 2, ..., N/2.  Every element is
 * summed as a butterfly: pairs at distance N/2 first, then N/4, ..., each
 * partial rounded to the storage type.  VRC_HD and VRC_HD_ORDER return the
 * same bits.
 *   VRC_HD            one launch per step: 2 log2 N launches for the
 *                     all-reduce, log2 N for the all-gather.  The stand-alone
 *                     reduce-scatter has no room for the N/2 blocks of
 *                     partials each rank holds after its first step (the
 *                     library allocates nothing), so it runs as VRC_HD_ORDER.
 *   VRC_HD_ORDER      one launch with the fused traffic, partials in
 *                     registers, in phases at 8 and 16 ranks as VRC_FUSED.
 *                     For the all-gather it equals VRC_FUSED.
 *                     At 2 ranks the butterfly is a single add rounded once,
 *                     bit for bit the rank-order fold, so it runs (and
 *                     vrc_plan reports it) as the fused kernel.
 * Size-based selection between the two step-by-step algorithms [TP]:
 *   VRC_SELECT        VRC_HD when nranks is a power of two and each rank's
 *                     input holds at most VRC_SELECT_HD_MAX_BYTES.  For the
 *                     all-gather at other rank counts, VRC_TREE while it
 *                     saves launches, L = (nranks-1) - 2 ceil(log2 nranks) >
 *                     0, and each rank's input holds at most
 *                     L * VRC_SELECT_TREE_BYTES_PER_SAVED_LAUNCH.  Else
 *                     VRC_RING.  The bits are those of the algorithm chosen
 *                     (vrc_plan shows which: 2 log2 N or 2(N-1) launches for
 *                     the all-reduce).  Any nranks is accepted.  The limits
 *                     are where the ring's fewer, larger launches overtake
 *                     the log-depth algorithms on MI355X (8 ranks:
 *                     halving-doubling 8 % faster at 16 MiB, the ring 3 %
 *                     faster at 128 MiB per rank; the tree all-gather 13-35 %
 *                     faster than the ring at 10-14 ranks and 64 KiB, within
 *                     5 % either way at 128-512 KiB, slower from 1 MiB). */
/* Binomial tree [TREE], all-gather only (vrc_allreduce and
 * vrc_reduce_scatter return VRC_ERR_UNSUPPORTED for it): the textbook
 * binomial gather to rank 0 followed by the binomial broadcast from rank 0
 * (Thakur, Rabenseifner and Gropp, "Optimization of Collective Communication
 * Operations in MPICH", IJHPCA 2005).  Gather step with distance d = 1, 2,
 * 4, ... (< nranks): rank r with r mod 2d == d hands the slabs it holds,
 * [r, min(r+d, nranks)), to rank r-d.  Broadcast steps with the distances in
 * reverse: rank r with r mod 2d == 0 copies its whole output to rank r+d.
 *   VRC_TREE          one launch per step: 2 ceil(log2 nranks) launches, any
 *                     nranks.  The bytes are the concatenation, as in every
 *                     all-gather mode. */
#define VRC_SELECT_HD_MAX_BYTES (64ull << 20)
#define VRC_SELECT_TREE_BYTES_PER_SAVED_LAUNCH (128ull << 10)
typedef enum {
    VRC_RING = 0,
    VRC_FUSED = 1,
    VRC_RING_CHAINED = 2,
    VRC_RING_ORDER = 3,
    VRC_HD = 4,
    VRC_HD_ORDER = 5,
    VRC_SELECT = 6,
    VRC_TREE = 7
} vrc_mode_t;

typedef enum {
    VRC_OK = 0,
    VRC_ERR_INVALID_ARG = 1, /* null array/pointer, nranks out of range, bad shape */
    VRC_ERR_UNSUPPORTED = 2, /* unknown dtype, op or mode */
    VRC_ERR_ALIAS = 3,       /* buffers overlap in a way the call does not allow */
    VRC_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} vrc_status_t;

/*
 * All-reduce (sum) [RS][RING][NAIVE][TP].
 *   recv[r][i] = sum over ranks q of send[q][i], for every rank r.
 *   send[r], recv[r]: `count` elements each, flat.
 *   nranks in [1, VRC_MAX_RANKS].  nranks == 1 copies (no-op in place).
 *   In place is allowed per rank (recv[r] == send[r]); any other overlap
 *   between a recv buffer and any other buffer returns VRC_ERR_ALIAS.
 *   VRC_RING enqueues 2*(nranks-1) kernels (nranks-1 adds, nranks-1 copies);
 *   VRC_FUSED enqueues one.
 *   count == 0 returns VRC_OK and enqueues nothing (null pointers allowed).
 */
vrc_status_t vrc_allreduce(const void* const* send, void* const* recv, int nranks, size_t count,
                           vrc_dtype_t dtype, vrc_op_t op, vrc_mode_t mode, vrc_stream_t stream);

/*
 * Bucketed all-reduce, overlapped with the computation that produces its
 * input [OVERLAP] (www.bjdmk.com.cn/news/5966809/, sections 4.2 and 4.3:
 * the compute stream records an event when a chunk of the tensor is ready,
 * the communication stream waits on that event and all-reduces the chunk
 * while the next chunk is computed).
 *   Every rank's buffer is cut into buckets of `bucket` elements (the last
 *   one holds the rest): bucket k is elements [k*bucket, min((k+1)*bucket,
 *   count)).  For k = 0, 1, ... the call enqueues on `stream` a wait on
 *   ready[k] (when `ready` is not NULL) and then the all-reduce of bucket k
 *   alone, exactly as vrc_allreduce would run it on those slices, and
 *   VRC_SELECT picks per bucket.  VRC_FUSED and the halving-doubling modes
 *   fold every element the same way whatever the partition, so they give
 *   the bits of the unbucketed call; the ring modes fold chunk c of each
 *   bucket from rank c, so theirs are the bits of each bucket's own ring.
 *   ready     NULL, or `nready` == number of buckets events (hipEvent_t)
 *             recorded by the caller on the stream that produces the data;
 *             NULL with nready == 0 runs the buckets back to back.
 *   The buffers, in-place rule, modes and errors are those of
 *   vrc_allreduce over the whole buffers (VRC_TREE is refused); bucket == 0,
 *   a NULL event or a wrong nready returns VRC_ERR_INVALID_ARG before
 *   anything is enqueued.  A HIP failure at bucket k returns VRC_ERR_HIP
 *   with buckets 0..k-1 already enqueued.  count == 0 enqueues nothing.
 */
vrc_status_t vrc_allreduce_bucketed(const void* const* send, void* const* recv, int nranks, size_t count,
                                    vrc_dtype_t dtype, vrc_op_t op, vrc_mode_t mode, size_t bucket,
                                    const vrc_event_t* ready, int nready, vrc_stream_t stream);

/*
 * Reduce-scatter (sum) [RS][REM][TP].
 *   Each send[r] holds `count` elements viewed as [outer, count/outer].
 *   outer == 1: recv[c] receives the reduced flat chunk c (its length is the
 *               chunk length above; the last rank takes the remainder).
 *   outer  > 1: (count/outer) must be divisible by nranks; chunk c is the
 *               column block [c*w, (c+1)*w) of every row, w = count/outer/
 *               nranks, and recv[c] is [outer, w] row-major.  This is the
 *               reduce-scatter of a tensor along a dimension, with outer =
 *               the product of the sizes before that dimension.
 *   VRC_RING adds the chunk in the ring order ((x_c + x_{c+1}) + ...) and
 *   keeps the running partial of chunk c in recv[c] (nranks-1 launches).
 *   VRC_FUSED folds x_0 + ... + x_{N-1} in fp32 and rounds once (1 launch).
 *   recv buffers must not overlap each other or any send buffer.
 */
vrc_status_t vrc_reduce_scatter(const void* const* send, void* const* recv, int nranks,
                                size_t count, size_t outer, vrc_dtype_t dtype, vrc_op_t op,
                                vrc_mode_t mode, vrc_stream_t stream);

/*
 * All-gather [RING][INFER][TP].
 *   Each send[r] holds `count` elements viewed as [outer, row], row =
 *   count/outer.  Each recv[r] is [outer, nranks*row]: rank q's input lands
 *   in columns [q*row, (q+1)*row).  outer == 1 is plain concatenation; outer
 *   > 1 is concatenation along a dimension (outer = product of the sizes
 *   before it).  Every rank receives the same bytes.
 *   VRC_RING relays slabs around the ring (nranks-1 launches: rank r copies
 *   slab (r-1-s) from rank r-1 at step s, and its own slab in step 0).
 *   VRC_FUSED reads each input once and writes it to all outputs.
 *   VRC_TREE gathers the slabs to rank 0 and broadcasts them along a
 *   binomial tree (2 ceil(log2 nranks) launches).
 *   recv buffers must not overlap each other or any send buffer.
 */
vrc_status_t vrc_all_gather(const void* const* send, void* const* recv, int nranks, size_t count,
                            size_t outer, vrc_dtype_t dtype, vrc_mode_t mode, vrc_stream_t stream);

/*
 * Launch plan, host only: what a call would enqueue, without touching the
 * GPU.  vrc_plan takes the arguments of the collective named by `coll`
 * (`outer` is ignored for the all-reduce and is the bucket size for
 * VRC_COLL_ALLREDUCE_BUCKETED, planned without events) and fills `ops` with one entry
 * per operation, in launch order.  Ring and halving-doubling steps give one
 * entry per rank operation of the step (VRC_OP_ADD: d = a + b, VRC_OP_COPY:
 * d = a, over `rows` rows of `width` elements with the given row strides in
 * elements; a, b and d point at element (0,0) of the operands inside the
 * caller's buffers).  Single-launch kernels give one entry per launch with
 * only `kind`, `launch`, width = count and the launch geometry set.  Arguments are validated as
 * in the real call.  If more than `cap` entries are needed the first `cap`
 * are written, *n_ops receives the full count and VRC_ERR_INVALID_ARG is
 * returned.  Used by the tests to check the schedules on the CPU, and for
 * debugging.
 */
typedef enum {
    VRC_COLL_ALLREDUCE = 0,
    VRC_COLL_REDUCE_SCATTER = 1,
    VRC_COLL_ALL_GATHER = 2,
    VRC_COLL_ALLREDUCE_BUCKETED = 3 /* `outer` carries the bucket size in elements; no events */
} vrc_coll_t;

typedef enum {
    VRC_OP_ADD = 0,
    VRC_OP_COPY = 1,
    VRC_OP_FUSED_ALLREDUCE = 2,
    VRC_OP_FUSED_REDUCE_SCATTER = 3,
    VRC_OP_FUSED_ALL_GATHER = 4,
    VRC_OP_CHAIN_ALLREDUCE = 5,      /* VRC_RING_CHAINED */
    VRC_OP_CHAIN_REDUCE_SCATTER = 6,
    VRC_OP_CHAIN_ALL_GATHER = 7,
    VRC_OP_RING_ORDER_ALLREDUCE = 8, /* VRC_RING_ORDER */
    VRC_OP_RING_ORDER_REDUCE_SCATTER = 9,
    VRC_OP_BUTTERFLY_ALLREDUCE = 10, /* VRC_HD_ORDER */
    VRC_OP_BUTTERFLY_REDUCE_SCATTER = 11,
    VRC_OP_FUSED_ALLREDUCE_REALIGNED = 12,   /* VRC_FUSED, outputs on different 128-byte offsets */
    VRC_OP_BUTTERFLY_ALLREDUCE_REALIGNED = 13, /* VRC_HD_ORDER, outputs on different 128-byte offsets */
    VRC_OP_RING_ORDER_ALLREDUCE_REALIGNED = 14, /* VRC_RING_ORDER, outputs on different 128-byte offsets */
    VRC_OP_FUSED_ALLREDUCE_PHASED = 15,     /* VRC_FUSED, large calls from 6 ranks: read, then write, by phases */
    VRC_OP_BUTTERFLY_ALLREDUCE_PHASED = 16, /* VRC_HD_ORDER, the same at 8 and 16 ranks */
    VRC_OP_RING_ORDER_ALLREDUCE_PHASED = 17 /* VRC_RING_ORDER, the same from 6 ranks */
} vrc_op_kind_t;

typedef struct {
    int launch;            /* index of the kernel launch this operation belongs to */
    int kind;              /* vrc_op_kind_t */
    const void* a;         /* first operand, element (0,0) */
    const void* b;         /* second operand (VRC_OP_ADD only) */
    void* d;               /* destination */
    size_t rows, width;    /* elements */
    size_t stride_a, stride_b, stride_d; /* row strides, elements (rows > 1) */
    /* Launch geometry of the kernel launch, the same in every entry of one
     * launch, computed for a device of 256 CUs (MI355X; a real call uses the
     * device's own CU count): workgroups in x and y, lanes per workgroup, and
     * 16-byte vectors per rank (per operand for a ring step) that a lane of
     * the main loop keeps in flight. */
    unsigned grid_x, grid_y, block, vectors;
} vrc_op_desc;

vrc_status_t vrc_plan(vrc_coll_t coll, const void* const* send, void* const* recv, int nranks, size_t count,
                      size_t outer, vrc_dtype_t dtype, vrc_mode_t mode, vrc_op_desc* ops, int cap, int* n_ops,
                      int* n_launches);

/* Offset and length (elements) of chunk `chunk` of a flat buffer of `count`
 * elements split over `nranks` [REM].  Host-only; touches no GPU. */
vrc_status_t vrc_chunk_range(size_t count, int nranks, int chunk, size_t* offset, size_t* length);

/* Static, human-readable text for a status code. */
const char* vrc_status_string(vrc_status_t status);

/* HIP error code of the most recent VRC_ERR_HIP on the calling thread (0 if none). */
int vrc_last_hip_error(void);

/* VRC_VERSION of the loaded library. */
int vrc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VRC_H */
