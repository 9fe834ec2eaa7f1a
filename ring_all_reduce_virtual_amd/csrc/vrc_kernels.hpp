// vrc_kernels.hpp -- HIP kernels (gfx950) for the virtual-rank collectives.
//
// All kernels are bandwidth-bound streaming loops: 256-lane workgroups (four
// wave64s), a grid sized to the CU count, grid-stride iteration over 16-byte
// vectors, and a scalar pass for the elements before the first 16-byte
// boundary and after the last one.  No MFMA: the work is a sum, not a
// contraction.
//
// Geometry.  An operand region is `rows` rows of `width` elements with a row
// stride in elements.  The host splits each row into `head` scalar elements
// (up to the first 16-byte boundary), `nvb` 16-byte vectors and `tail`
// scalar elements; when the operands of one region do not share the same
// address offset modulo 16 (or a row stride is not a multiple of 16 bytes)
// it sets head = width, nvb = tail = 0 and the region runs scalar.
#pragma once

#include "vrc_elem.hpp"

namespace vrc {

constexpr int kBlock = 256;
constexpr int kMaxRanks = 16;
constexpr int kMaxStepOps = 2 * kMaxRanks;

struct RowSplit {
    uint64_t head, nvb, tail;
};

// Map a scalar slot k (0 <= k < rows*(head+tail)) to (row, column).
__device__ __forceinline__ void scalar_slot(uint64_t k, const RowSplit& g, uint64_t vec, uint64_t& row,
                                            uint64_t& col)
{
    const uint64_t per_row = g.head + g.tail;
    row = k / per_row;
    const uint64_t j = k - row * per_row;
    col = (j < g.head) ? j : g.head + g.nvb * vec + (j - g.head);
}

// ---------------------------------------------------------------------------
// Ring step: one launch runs one reduce-scatter step (d = a + b) or one
// all-gather step (d = a) for every rank at once; blockIdx.y is the rank's
// operation.
// ---------------------------------------------------------------------------
struct StepOp {
    const char* a;  // element (0,0) of the first operand region
    const char* b;  // second operand (add only)
    char* d;        // destination
    uint64_t rows, width;
    uint64_t sa, sb, sd;  // row strides, elements
    RowSplit g;
};

struct StepArgs {
    StepOp op[kMaxStepOps];
};

template <class T, bool ADD, bool NT>
__global__ __launch_bounds__(kBlock) void k_ring_step(StepArgs args)
{
    const StepOp& op = args.op[blockIdx.y];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;

    const uint64_t nv = op.rows * op.g.nvb;
    const uint64_t body = op.g.head * E;
    if (op.rows == 1) {
        for (uint64_t v = tid; v < nv; v += nthreads) {
            const uint64_t off = body + v * 16;
            u32x4 x = ld16<NT>(op.a + off);
            if constexpr (ADD) x = add_v<T>(x, ld16<NT>(op.b + off));
            st16<NT>(op.d + off, x);
        }
    } else {
        for (uint64_t v = tid; v < nv; v += nthreads) {
            const uint64_t row = v / op.g.nvb;
            const uint64_t col = (v - row * op.g.nvb) * 16 + body;
            u32x4 x = ld16<NT>(op.a + row * op.sa * E + col);
            if constexpr (ADD) x = add_v<T>(x, ld16<NT>(op.b + row * op.sb * E + col));
            st16<NT>(op.d + row * op.sd * E + col, x);
        }
    }

    const uint64_t ns = op.rows * (op.g.head + op.g.tail);
    for (uint64_t k = tid; k < ns; k += nthreads) {
        uint64_t row, col;
        scalar_slot(k, op.g, T::VEC, row, col);
        typename T::S x = load_s<T>(op.a + (row * op.sa + col) * E);
        if constexpr (ADD) x = add_s<T>(x, load_s<T>(op.b + (row * op.sb + col) * E));
        store_s<T>(op.d + (row * op.sd + col) * E, x);
    }
}

// ---------------------------------------------------------------------------
// Fused all-reduce: every lane reads element block i of all N inputs, folds
// them in rank order in the accumulator, rounds once and writes the result
// to all N outputs.  Reads precede writes within a lane, so in-place calls
// are safe.  U independent vectors per lane per iteration keep U*N 16-byte
// loads in flight.
// ---------------------------------------------------------------------------
struct FusedArArgs {
    const char* src[kMaxRanks];
    char* dst[kMaxRanks];
    uint64_t count;  // elements per rank
    RowSplit g;      // one row of `count` elements
};

template <class T, int N>
__device__ __forceinline__ u32x4 fold_v(const u32x4* in)
{
    typename T::A acc[T::VEC], x[T::VEC];
    T::unpack(in[0], acc);
#pragma unroll
    for (int r = 1; r < N; r++) {
        T::unpack(in[r], x);
#pragma unroll
        for (int i = 0; i < T::VEC; i++) acc[i] = T::add(acc[i], x[i]);
    }
    return T::pack(acc);
}

// How the fused kernels combine the N values of one element.
//  RankFold:  x_0 + x_1 + ... + x_{N-1} folded left in the accumulator type,
//             rounded once (the collector all-reduce).
//  Butterfly: halving-doubling order, N a power of two: pairs at distance
//             N/2 first, then N/4, ..., each partial rounded to the storage
//             type: v[r] = v[r] (+) v[r + d] for r < d, d = N/2 .. 1.
struct RankFold {
    template <class T, int N>
    __device__ static u32x4 vec(u32x4* in) { return fold_v<T, N>(in); }
    template <class T, int N>
    __device__ static typename T::S scalar(typename T::S* in)
    {
        typename T::A acc = T::widen(in[0]);
#pragma unroll
        for (int r = 1; r < N; r++) acc = T::add(acc, T::widen(in[r]));
        return T::narrow(acc);
    }
};

struct Butterfly {
    template <class T, int N>
    __device__ static u32x4 vec(u32x4* in)
    {
        static_assert((N & (N - 1)) == 0, "butterfly needs a power of two");
#pragma unroll
        for (int d = N / 2; d >= 1; d /= 2)
#pragma unroll
            for (int r = 0; r < d; r++) in[r] = add_v<T>(in[r], in[r + d]);
        return in[0];
    }
    template <class T, int N>
    __device__ static typename T::S scalar(typename T::S* in)
    {
#pragma unroll
        for (int d = N / 2; d >= 1; d /= 2)
#pragma unroll
            for (int r = 0; r < d; r++) in[r] = add_s<T>(in[r], in[r + d]);
        return in[0];
    }
};

template <class T, int N, int U, bool NT, class Fold = RankFold>
__global__ __launch_bounds__(kBlock) void k_fused_allreduce(FusedArArgs a)
{
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const uint64_t body = a.g.head * E;
    const uint64_t nv = a.g.nvb;

    uint64_t v = tid;
    if constexpr (U > 1) {
        for (; v + (U - 1) * nthreads < nv; v += U * nthreads) {
            u32x4 in[U][N];
#pragma unroll
            for (int u = 0; u < U; u++)
#pragma unroll
                for (int r = 0; r < N; r++) in[u][r] = ld16<NT>(a.src[r] + body + (v + u * nthreads) * 16);
#pragma unroll
            for (int u = 0; u < U; u++) {
                const u32x4 s = Fold::template vec<T, N>(in[u]);
#pragma unroll
                for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + (v + u * nthreads) * 16, s);
            }
        }
    }
    for (; v < nv; v += nthreads) {
        u32x4 in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + body + v * 16);
        const u32x4 s = Fold::template vec<T, N>(in);
#pragma unroll
        for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + v * 16, s);
    }

    const uint64_t ns = a.g.head + a.g.tail;
    for (uint64_t k = tid; k < ns; k += nthreads) {
        const uint64_t i = (k < a.g.head) ? k : a.g.head + a.g.nvb * T::VEC + (k - a.g.head);
        typename T::S in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = load_s<T>(a.src[r] + i * E);
        const typename T::S s = Fold::template scalar<T, N>(in);
#pragma unroll
        for (int r = 0; r < N; r++) store_s<T>(a.dst[r] + i * E, s);
    }
}

// ---------------------------------------------------------------------------
// Fused reduce-scatter: blockIdx.y = chunk c.  Output c is the rank-order
// fold of chunk c over all N inputs, rounded once.
// ---------------------------------------------------------------------------
struct RsChunk {
    uint64_t src_off;  // element offset of chunk c's (0,0) in every input
    char* d;           // output c
    uint64_t rows, width;
    uint64_t s_src, s_dst;  // row strides, elements
    RowSplit g;
};

struct FusedRsArgs {
    const char* src[kMaxRanks];
    RsChunk ch[kMaxRanks];
};

template <class T, int N, bool NT, class Fold = RankFold>
__global__ __launch_bounds__(kBlock) void k_fused_reduce_scatter(FusedRsArgs a)
{
    const RsChunk& c = a.ch[blockIdx.y];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const uint64_t nv = c.rows * c.g.nvb;
    for (uint64_t v = tid; v < nv; v += nthreads) {
        const uint64_t row = (c.rows == 1) ? 0 : v / c.g.nvb;
        const uint64_t col = (v - row * c.g.nvb) * 16 + c.g.head * E;
        const uint64_t so = (c.src_off + row * c.s_src) * E + col;
        u32x4 in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + so);
        st16<NT>(c.d + row * c.s_dst * E + col, Fold::template vec<T, N>(in));
    }
    const uint64_t ns = c.rows * (c.g.head + c.g.tail);
    for (uint64_t k = tid; k < ns; k += nthreads) {
        uint64_t row, col;
        scalar_slot(k, c.g, T::VEC, row, col);
        const uint64_t so = (c.src_off + row * c.s_src + col) * E;
        typename T::S in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = load_s<T>(a.src[r] + so);
        store_s<T>(c.d + (row * c.s_dst + col) * E, Fold::template scalar<T, N>(in));
    }
}

// ---------------------------------------------------------------------------
// Fused all-gather: blockIdx.y = source rank q.  Input q ([rows, width]) is
// read once and written into column slab q of every output ([rows,
// n*width]).
// ---------------------------------------------------------------------------
struct FusedAgArgs {
    const char* src[kMaxRanks];
    char* dst[kMaxRanks];
    uint64_t rows, width;  // input geometry; output row stride is n * width
    int n;
    RowSplit g[kMaxRanks];  // per source rank (its slab offset sets the alignment)
};

template <class T, bool NT>
__global__ __launch_bounds__(kBlock) void k_fused_all_gather(FusedAgArgs a)
{
    const int q = blockIdx.y;
    const RowSplit& g = a.g[q];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const uint64_t s_dst = (uint64_t)a.n * a.width;
    const uint64_t slab = (uint64_t)q * a.width;
    const uint64_t nv = a.rows * g.nvb;
    for (uint64_t v = tid; v < nv; v += nthreads) {
        const uint64_t row = (a.rows == 1) ? 0 : v / g.nvb;
        const uint64_t col = (v - row * g.nvb) * 16 + g.head * E;
        const u32x4 x = ld16<NT>(a.src[q] + row * a.width * E + col);
        const uint64_t dof = (row * s_dst + slab) * E + col;
        for (int r = 0; r < a.n; r++) st16<NT>(a.dst[r] + dof, x);
    }
    const uint64_t ns = a.rows * (g.head + g.tail);
    for (uint64_t k = tid; k < ns; k += nthreads) {
        uint64_t row, col;
        scalar_slot(k, g, T::VEC, row, col);
        const typename T::S x = load_s<T>(a.src[q] + (row * a.width + col) * E);
        const uint64_t dof = (row * s_dst + slab + col) * E;
        for (int r = 0; r < a.n; r++) store_s<T>(a.dst[r] + dof, x);
    }
}

// ---------------------------------------------------------------------------
// Single-launch ring.  In the ring schedule element i of chunk c depends only
// on element i of chunk c at the previous step: the reduce-scatter carries
// the partial of chunk c from rank c+1 to c+2 ... to c+N-1 (= c-1), and the
// all-gather relays the finished chunk from rank c-1 to c, c+1, ..., c+N-2.
// Each element is therefore an independent chain of 2(N-1) operations, and
// one launch can run every chain to the end with no grid-wide barrier.
// blockIdx.y = chunk c, so the rank rotation is uniform per workgroup.
//
// MEM = true ("chained"): every step writes its partial into the next
// rank's buffer and the following step reads it back from there, so the
// reads and writes per step are those of the per-step ring launches.
// MEM = false ("ring order"): the partial stays in registers; every input is
// read once and every output written once (the fused kernel's traffic), with
// the ring's summation order and per-step rounding.  Both give the per-step
// ring's bits.
// ---------------------------------------------------------------------------
struct ChainChunk {
    uint64_t off;          // element offset of chunk (0,0) in every rank buffer
    uint64_t rows, width;  // chunk geometry
    uint64_t stride;       // row stride of the rank buffers, elements
    RowSplit g;
};

struct ChainArgs {
    const char* src[kMaxRanks];
    char* dst[kMaxRanks];
    ChainChunk ch[kMaxRanks];
};

// All-reduce chain over flat chunks (rows == 1).
template <class T, int N, bool MEM, bool NT>
__global__ __launch_bounds__(kBlock) void k_ring_chain_allreduce(ChainArgs a)
{
    const int c = blockIdx.y;
    const ChainChunk& k = a.ch[c];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const int owner = (c + N - 1) % N;  // holds chunk c complete after the reduce-scatter
    const uint64_t body = (k.off + k.g.head) * E;
    for (uint64_t v = tid; v < k.g.nvb; v += nthreads) {
        const uint64_t o = body + v * 16;
        u32x4 p;
        if constexpr (MEM) {
            p = ld16<NT>(a.src[c] + o);
#pragma unroll
            for (int t = 1; t < N; t++) {
                const int r = (c + t) % N;
                const u32x4 own = ld16<NT>(a.src[r] + o);
                if (t > 1) p = ld16<NT>(a.dst[(c + t - 1) % N] + o);
                p = add_v<T>(p, own);
                st16<NT>(a.dst[r] + o, p);
            }
#pragma unroll
            for (int s = 0; s < N - 1; s++) {
                const int r = (c + s) % N;
                st16<NT>(a.dst[r] + o, ld16<NT>(a.dst[(c + s + N - 1) % N] + o));
            }
        } else {
            u32x4 in[N];
#pragma unroll
            for (int t = 0; t < N; t++) in[t] = ld16<NT>(a.src[(c + t) % N] + o);
            p = in[0];
#pragma unroll
            for (int t = 1; t < N; t++) p = add_v<T>(p, in[t]);
#pragma unroll
            for (int t = 0; t < N; t++) st16<NT>(a.dst[(owner + 1 + t) % N] + o, p);
        }
    }
    const uint64_t ns = k.g.head + k.g.tail;
    for (uint64_t j = tid; j < ns; j += nthreads) {
        const uint64_t col = (j < k.g.head) ? j : k.g.head + k.g.nvb * T::VEC + (j - k.g.head);
        const uint64_t o = (k.off + col) * E;
        typename T::S p = load_s<T>(a.src[c] + o);
        if constexpr (MEM) {
#pragma unroll
            for (int t = 1; t < N; t++) {
                const int r = (c + t) % N;
                const typename T::S own = load_s<T>(a.src[r] + o);
                if (t > 1) p = load_s<T>(a.dst[(c + t - 1) % N] + o);
                p = add_s<T>(p, own);
                store_s<T>(a.dst[r] + o, p);
            }
#pragma unroll
            for (int s = 0; s < N - 1; s++)
                store_s<T>(a.dst[(c + s) % N] + o, load_s<T>(a.dst[(c + s + N - 1) % N] + o));
        } else {
            typename T::S in[N];
#pragma unroll
            for (int t = 0; t < N; t++) in[t] = load_s<T>(a.src[(c + t) % N] + o);
#pragma unroll
            for (int t = 1; t < N; t++) p = add_s<T>(p, in[t]);
#pragma unroll
            for (int t = 0; t < N; t++) store_s<T>(a.dst[(owner + 1 + t) % N] + o, p);
        }
    }
}

// Reduce-scatter chain: chunk c of every rank ([rows, width] with row stride
// `stride`) is summed in ring order into output c ([rows, width], dense).
template <class T, int N, bool MEM, bool NT>
__global__ __launch_bounds__(kBlock) void k_ring_chain_reduce_scatter(ChainArgs a)
{
    const int c = blockIdx.y;
    const ChainChunk& k = a.ch[c];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    char* out = a.dst[c];
    const uint64_t nv = k.rows * k.g.nvb;
    for (uint64_t v = tid; v < nv; v += nthreads) {
        const uint64_t row = (k.rows == 1) ? 0 : v / k.g.nvb;
        const uint64_t col = (v - row * k.g.nvb) * 16 + k.g.head * E;
        const uint64_t so = (k.off + row * k.stride) * E + col;
        const uint64_t dof = row * k.width * E + col;
        u32x4 p;
        if constexpr (MEM) {
            p = ld16<NT>(a.src[c] + so);
#pragma unroll
            for (int t = 1; t < N; t++) {
                const u32x4 own = ld16<NT>(a.src[(c + t) % N] + so);
                if (t > 1) p = ld16<NT>(out + dof);
                p = add_v<T>(p, own);
                st16<NT>(out + dof, p);
            }
        } else {
            u32x4 in[N];
#pragma unroll
            for (int t = 0; t < N; t++) in[t] = ld16<NT>(a.src[(c + t) % N] + so);
            p = in[0];
#pragma unroll
            for (int t = 1; t < N; t++) p = add_v<T>(p, in[t]);
            st16<NT>(out + dof, p);
        }
    }
    const uint64_t ns = k.rows * (k.g.head + k.g.tail);
    for (uint64_t j = tid; j < ns; j += nthreads) {
        uint64_t row, col;
        scalar_slot(j, k.g, T::VEC, row, col);
        const uint64_t so = (k.off + row * k.stride + col) * E;
        const uint64_t dof = (row * k.width + col) * E;
        typename T::S p = load_s<T>(a.src[c] + so);
#pragma unroll
        for (int t = 1; t < N; t++) {
            const typename T::S own = load_s<T>(a.src[(c + t) % N] + so);
            if (MEM && t > 1) p = load_s<T>(out + dof);
            p = add_s<T>(p, own);
            if (MEM || t == N - 1) store_s<T>(out + dof, p);
        }
    }
}

// All-gather chain (memory-faithful relay): slab q (blockIdx.y) is copied
// from input q into output q and output q+1, then relayed output q+t-1 ->
// output q+t for t = 2..N-1.  Inputs are [rows, width]; outputs are
// [rows, N*width] with slab q at column q*width.
template <class T, int N, bool NT>
__global__ __launch_bounds__(kBlock) void k_ring_chain_all_gather(FusedAgArgs a)
{
    const int q = blockIdx.y;
    const RowSplit& g = a.g[q];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const uint64_t s_dst = (uint64_t)N * a.width;
    const uint64_t slab = (uint64_t)q * a.width;
    const uint64_t nv = a.rows * g.nvb;
    for (uint64_t v = tid; v < nv; v += nthreads) {
        const uint64_t row = (a.rows == 1) ? 0 : v / g.nvb;
        const uint64_t col = (v - row * g.nvb) * 16 + g.head * E;
        const uint64_t dof = (row * s_dst + slab) * E + col;
        const u32x4 x = ld16<NT>(a.src[q] + row * a.width * E + col);
        st16<NT>(a.dst[q] + dof, x);
        if (N > 1) st16<NT>(a.dst[(q + 1) % N] + dof, x);
#pragma unroll
        for (int t = 2; t < N; t++) st16<NT>(a.dst[(q + t) % N] + dof, ld16<NT>(a.dst[(q + t - 1) % N] + dof));
    }
    const uint64_t ns = a.rows * (g.head + g.tail);
    for (uint64_t j = tid; j < ns; j += nthreads) {
        uint64_t row, col;
        scalar_slot(j, g, T::VEC, row, col);
        const uint64_t dof = (row * s_dst + slab + col) * E;
        const typename T::S x = load_s<T>(a.src[q] + (row * a.width + col) * E);
        store_s<T>(a.dst[q] + dof, x);
        if (N > 1) store_s<T>(a.dst[(q + 1) % N] + dof, x);
#pragma unroll
        for (int t = 2; t < N; t++) store_s<T>(a.dst[(q + t) % N] + dof, load_s<T>(a.dst[(q + t - 1) % N] + dof));
    }
}

}  // namespace vrc
