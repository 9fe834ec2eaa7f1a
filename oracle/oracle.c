/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the ring
 * all-reduce and its reduce-scatter and all-gather halves over N virtual
 * ranks.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code,
 * header, table or helper with the HIP library; the product path never
 * calls it.
 *
 * Sources (pages are named by address; sections by their heading):
 *  [RS]   ai6s.net/6a102b5410ee7a33f2746c06.html, section "hcomm 与 HCCL 的
 *         关系" (how HCCL splits AllReduce into ReduceScatter + AllGather) and
 *         its simplified ReduceScatter listing: cut the buffer into nranks
 *         chunks; at every step send one chunk to the next rank, receive one
 *         chunk from the previous rank, add the received chunk element-wise,
 *         then move both chunk indices one down (mod nranks).
 *  [RING] hwcomputing.csdn.net/6a0dc11a10ee7a33f273f7fd.html, section "Ring
 *         通信为什么常见" (4-card walkthrough): logical ring 0->1->..->N-1->0;
 *         in the first step card r hands block r to card r+1; each card adds
 *         what it received and passes the result on; after N-1 such steps
 *         each card owns one complete block; the all-gather phase then relays
 *         the complete blocks in N-1 copy steps.  Per-card traffic is
 *         2(N-1)*S/N.
 *  [REM]  ai6s.net/6a157e6510ee7a33f27553e9.html, section "自定义通信模式"
 *         (custom all-gather listing): equal chunks, the last chunk takes the
 *         remainder.
 *  [NAIVE] hwcomputing.csdn.net/6a0dc11a10ee7a33f273f7fd.html, section "为什么
 *         大模型训练离不开通信": the naive all-reduce, where one collector adds
 *         every contribution and hands the sum back to all ranks.
 *  [HD]   ai6s.net/6a0dd5b5662f9a54cb75ef90.html, section "TP 通信": on fully
 *         connected NPUs the all-reduce uses halving-doubling, finishing in a
 *         logarithmic number of steps.  The pages give no further detail; the
 *         oracle follows the textbook algorithm (recursive halving
 *         reduce-scatter, then recursive doubling all-gather, for N a power of
 *         two; Thakur, Rabenseifner and Gropp, "Optimization of Collective
 *         Communication Operations in MPICH", IJHPCA 19(1), 2005): at the step
 *         with distance d (N/2, N/4, ..., 1) rank r exchanges with r XOR d,
 *         keeps the half of its current block range that holds block r and
 *         adds the partner's copy of that half; the all-gather then doubles
 *         the owned range with distances 1, 2, ..., N/2.

 *  [TREE] ai6s.net/6a102b5410ee7a33f2746c06.html, sections "分布式推理中的通信"
 *         and "hcomm 在推理场景中的使用": the all-gather comes in a ring form
 *         and a tree form, chosen by data size.  The tree is not defined
 *         there; the oracle takes the textbook binomial tree (Thakur,
 *         Rabenseifner and Gropp 2005, binomial gather and binomial
 *         broadcast; all-gather = gather to rank 0, then broadcast from it):
 *         gather with distances d = 1, 2, 4, ... (< N), rank r with
 *         r mod 2d == d sending the slabs it holds, [r, min(r+d, N)), to rank
 *         r - d; then broadcast with the same distances in reverse order,
 *         rank r with r mod 2d == 0 sending all N slabs to rank r + d
 *         (if r + d < N).  2*ceil(log2 N) steps for any N.
 *
 * Readings taken where the pages are silent or garbled:
 *  - The listing adds into the chunk it sends; the walkthrough says a card
 *    adds what it received and passes that sum on.  The oracle adds the
 *    received payload into the receiving rank's copy of the received chunk.
 *  - "next" is rank r+1, "previous" is rank r-1 (mod N); the receive buffer
 *    is the message payload.
 *  - Element semantics: int32 adds wrap modulo 2^32; fp32 is one IEEE
 *    round-to-nearest-even add; fp16/bf16 widen exactly to fp32, add once in
 *    fp32, and round once to the storage format (ring partials travel in the
 *    storage format).  The fused all-reduce is the naive all-reduce: a left
 *    fold in rank order 0..N-1 in fp32 (uint32 for int32), rounded once.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math, no FTZ/DAZ).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Types and status codes                                              */
/* ------------------------------------------------------------------ */

enum { ORC_INT32 = 0, ORC_FP32 = 1, ORC_FP16 = 2, ORC_BF16 = 3 };

enum {
    ORC_OK = 0,
    ORC_E_ARG = 1,      /* bad arguments */
    ORC_E_NOMEM = 2,    /* malloc failed */
    ORC_E_EMPTY = 3,    /* a rank tried to receive from an empty inbox */
    ORC_E_TAG = 4,      /* a message carried the wrong source, phase, step or chunk */
    ORC_E_LEFTOVER = 5  /* messages left undelivered at the end */
};

enum {
    ORC_PHASE_RS = 0,
    ORC_PHASE_AG = 1,
    ORC_PHASE_HD_RS = 2,
    ORC_PHASE_HD_AG = 3,
    ORC_PHASE_TREE_GATHER = 4,
    ORC_PHASE_TREE_BCAST = 5
};

/* Test hook: plant one fault into the simulated transport. */
enum {
    ORC_FAULT_NONE = 0,
    ORC_FAULT_DROP = 1,      /* the message is never posted */
    ORC_FAULT_DUP = 2,       /* the message is posted twice */
    ORC_FAULT_MISROUTE = 3,  /* the message goes to rank r+2 instead of r+1 */
    ORC_FAULT_WRONG_CHUNK = 4 /* the sender sends its next chunk instead */
};

typedef struct {
    int kind;
    int phase;
    int step;
    int rank; /* sending rank */
} orc_fault;

/* One record per posted message, for schedule checks.  A message carries
 * the blocks [chunk, chunk_hi). */
typedef struct {
    int phase, step, src, dst, chunk;
    uint64_t elems;
    int chunk_hi;
} orc_msg_rec;

typedef struct {
    orc_msg_rec* log;     /* may be NULL */
    uint64_t log_cap;
    uint64_t log_len;
    uint64_t* sent_elems; /* per rank, may be NULL */
    uint64_t* recv_elems; /* per rank, may be NULL */
} orc_trace;

static size_t elem_size(int dt)
{
    switch (dt) {
    case ORC_INT32: return 4;
    case ORC_FP32: return 4;
    case ORC_FP16: return 2;
    case ORC_BF16: return 2;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* fp16 / bf16 codecs, written from the IEEE 754 binary format rules   */
/* ------------------------------------------------------------------ */

/* Decode a binary format with `ebits` exponent bits and `mbits` fraction
 * bits (sign in the top bit) into a float.  Every fp16 and bf16 value is
 * exactly representable as a float. */
static float small_decode(uint32_t bits, int ebits, int mbits)
{
    int bias = (1 << (ebits - 1)) - 1;
    uint32_t sign = (bits >> (ebits + mbits)) & 1u;
    uint32_t e = (bits >> mbits) & ((1u << ebits) - 1u);
    uint32_t m = bits & ((1u << mbits) - 1u);
    double v;
    if (e == 0) {
        v = ldexp((double)m, 1 - bias - mbits);                  /* zero / subnormal */
    } else if (e == (1u << ebits) - 1u) {
        v = (m == 0) ? INFINITY : NAN;                           /* inf / NaN */
    } else {
        v = ldexp((double)((1u << mbits) + m), (int)e - bias - mbits); /* normal */
    }
    return (float)(sign ? -v : v);
}

/* Round a float to the nearest value of the binary format (ties to even),
 * returning its bit pattern.  Overflow goes to infinity; NaN becomes the
 * format's quiet NaN with the input's sign. */
static uint32_t small_encode(float f, int ebits, int mbits)
{
    int bias = (1 << (ebits - 1)) - 1;
    int emin = 1 - bias;
    uint32_t sign = signbit(f) ? 1u : 0u;
    uint32_t sign_bits = sign << (ebits + mbits);
    uint32_t inf_bits = ((1u << ebits) - 1u) << mbits;
    double a = fabs((double)f);
    if (isnan(f)) return sign_bits | inf_bits | (1u << (mbits - 1));
    if (isinf(f)) return sign_bits | inf_bits;
    if (a == 0.0) return sign_bits;

    int e;
    frexp(a, &e);     /* a = m * 2^e with m in [0.5, 1) */
    e -= 1;           /* now a = m * 2^e with m in [1, 2) */
    if (e < emin) e = emin; /* subnormal range: fixed scale */

    /* Scale so that one unit is one ulp at exponent e, then round the
     * scaled value to an integer, ties to even (rint in the default
     * rounding mode).  Both steps are exact in double. */
    double q = ldexp(a, mbits - e);
    double r = rint(q);
    double two_m = ldexp(1.0, mbits);
    if (r >= 2.0 * two_m) { /* rounding carried into the next binade */
        r = r / 2.0;
        e += 1;
    }
    if (e > bias) return sign_bits | inf_bits; /* overflow */
    uint32_t ir = (uint32_t)r;
    if (r < two_m) return sign_bits | ir; /* subnormal (only when e == emin) */
    return sign_bits | ((uint32_t)(e + bias) << mbits) | (ir - (uint32_t)two_m);
}

static float f16_decode(uint16_t h) { return small_decode(h, 5, 10); }
static uint16_t f16_encode(float f) { return (uint16_t)small_encode(f, 5, 10); }
static float bf16_decode(uint16_t b) { return small_decode(b, 8, 7); }
static uint16_t bf16_encode(float f) { return (uint16_t)small_encode(f, 8, 7); }

/* ------------------------------------------------------------------ */
/* Element arithmetic in storage semantics                             */
/* ------------------------------------------------------------------ */

/* dst = a (+) b for one element of type dt (all three may alias). */
static void elem_add(int dt, void* dst, const void* a, const void* b)
{
    switch (dt) {
    case ORC_INT32: {
        uint32_t x, y, z;
        memcpy(&x, a, 4);
        memcpy(&y, b, 4);
        z = x + y; /* wraps modulo 2^32 */
        memcpy(dst, &z, 4);
        break;
    }
    case ORC_FP32: {
        float x, y, z;
        memcpy(&x, a, 4);
        memcpy(&y, b, 4);
        z = x + y;
        memcpy(dst, &z, 4);
        break;
    }
    case ORC_FP16: {
        uint16_t x, y, z;
        memcpy(&x, a, 2);
        memcpy(&y, b, 2);
        float s = f16_decode(x) + f16_decode(y);
        z = f16_encode(s);
        memcpy(dst, &z, 2);
        break;
    }
    case ORC_BF16: {
        uint16_t x, y, z;
        memcpy(&x, a, 2);
        memcpy(&y, b, 2);
        float s = bf16_decode(x) + bf16_decode(y);
        z = bf16_encode(s);
        memcpy(dst, &z, 2);
        break;
    }
    }
}

/* Accumulator for the fused (naive) all-reduce: fp32, or uint32 for int32. */
typedef struct {
    float f;
    uint32_t u;
} acc_t;

static void acc_set(int dt, acc_t* acc, const void* x)
{
    uint16_t h;
    switch (dt) {
    case ORC_INT32: memcpy(&acc->u, x, 4); break;
    case ORC_FP32: memcpy(&acc->f, x, 4); break;
    case ORC_FP16: memcpy(&h, x, 2); acc->f = f16_decode(h); break;
    case ORC_BF16: memcpy(&h, x, 2); acc->f = bf16_decode(h); break;
    }
}

static void acc_add(int dt, acc_t* acc, const void* x)
{
    uint16_t h;
    uint32_t u;
    float f;
    switch (dt) {
    case ORC_INT32: memcpy(&u, x, 4); acc->u = acc->u + u; break;
    case ORC_FP32: memcpy(&f, x, 4); acc->f = acc->f + f; break;
    case ORC_FP16: memcpy(&h, x, 2); acc->f = acc->f + f16_decode(h); break;
    case ORC_BF16: memcpy(&h, x, 2); acc->f = acc->f + bf16_decode(h); break;
    }
}

static void acc_store(int dt, const acc_t* acc, void* dst)
{
    uint16_t h;
    switch (dt) {
    case ORC_INT32: memcpy(dst, &acc->u, 4); break;
    case ORC_FP32: memcpy(dst, &acc->f, 4); break;
    case ORC_FP16: h = f16_encode(acc->f); memcpy(dst, &h, 2); break;
    case ORC_BF16: h = bf16_encode(acc->f); memcpy(dst, &h, 2); break;
    }
}

/* ------------------------------------------------------------------ */
/* Chunk geometry                                                      */
/* ------------------------------------------------------------------ */

/* A rank's buffer of `count` elements is viewed as [outer, row] with
 * row = count / outer.
 *  - outer == 1: chunk c is the contiguous range [c*base, (c+1)*base) with
 *    base = count / n, except that the last chunk runs to `count` [REM].
 *  - outer > 1: chunk c is the column block [c*w, (c+1)*w) of every row,
 *    with w = row / n (row must be divisible by n). */
typedef struct {
    uint64_t count, outer, row;
    int n;
} geom;

static uint64_t chunk_len(const geom* g, int c)
{
    if (g->outer == 1) {
        uint64_t base = g->count / (uint64_t)g->n;
        return (c == g->n - 1) ? g->count - base * (uint64_t)(g->n - 1) : base;
    }
    return g->outer * (g->row / (uint64_t)g->n);
}

/* Flat index, within a rank's buffer, of the k-th element of chunk c. */
static uint64_t chunk_elem(const geom* g, int c, uint64_t k)
{
    if (g->outer == 1) {
        uint64_t base = g->count / (uint64_t)g->n;
        return (uint64_t)c * base + k;
    }
    uint64_t w = g->row / (uint64_t)g->n;
    uint64_t o = k / w, j = k % w;
    return o * g->row + (uint64_t)c * w + j;
}

/* Chunk of a flat element index (outer == 1 only). */
static int chunk_of(uint64_t count, int n, uint64_t i)
{
    uint64_t base = count / (uint64_t)n;
    if (base == 0) return n - 1;
    uint64_t c = i / base;
    return (c >= (uint64_t)(n - 1)) ? n - 1 : (int)c;
}

static int mod(int a, int n) { return ((a % n) + n) % n; }

/* ------------------------------------------------------------------ */
/* Simulated transport: one FIFO inbox per rank                        */
/* ------------------------------------------------------------------ */

typedef struct msg {
    int src, phase, step, chunk, chunk_hi;
    uint64_t elems;
    unsigned char* payload;
    struct msg* next;
} msg;

typedef struct {
    msg* head;
    msg* tail;
} inbox;

typedef struct {
    int dt;
    int n;
    size_t esz;
    inbox* boxes;
    orc_trace* trace;
    const orc_fault* fault;
} net;

static void inbox_push(inbox* b, msg* m)
{
    m->next = NULL;
    if (b->tail) b->tail->next = m;
    else b->head = m;
    b->tail = m;
}

static msg* inbox_pop(inbox* b)
{
    msg* m = b->head;
    if (!m) return NULL;
    b->head = m->next;
    if (!b->head) b->tail = NULL;
    return m;
}

static void msg_free(msg* m)
{
    if (m) {
        free(m->payload);
        free(m);
    }
}

/* Copy `elems` elements (whose flat indices come from `idx_of`) out of a
 * rank's buffer into a fresh message. */
static msg* msg_make(const net* nt, int src, int phase, int step, int chunk,
                     const unsigned char* buf, uint64_t elems,
                     const geom* g, int slab_layout)
{
    msg* m = (msg*)calloc(1, sizeof(msg));
    if (!m) return NULL;
    m->payload = (unsigned char*)malloc(elems ? elems * nt->esz : 1);
    if (!m->payload) {
        free(m);
        return NULL;
    }
    m->src = src;
    m->phase = phase;
    m->step = step;
    m->chunk = chunk;
    m->chunk_hi = chunk + 1;
    m->elems = elems;
    for (uint64_t k = 0; k < elems; k++) {
        uint64_t at;
        if (slab_layout) { /* all-gather slab `chunk` of an [outer, n*row] buffer */
            uint64_t o = k / g->row, j = k % g->row;
            at = o * g->row * (uint64_t)g->n + (uint64_t)chunk * g->row + j;
        } else {
            at = chunk_elem(g, chunk, k);
        }
        memcpy(m->payload + k * nt->esz, buf + at * nt->esz, nt->esz);
    }
    return m;
}

/* Post a message to rank `dst`, applying a planted fault if one matches
 * (a misrouted message goes to dst+1). */
static int post_to(net* nt, msg* m, int dst)
{
    const orc_fault* f = nt->fault;
    int hit = f && f->kind != ORC_FAULT_NONE && f->phase == m->phase &&
              f->step == m->step && f->rank == m->src;
    if (hit && f->kind == ORC_FAULT_DROP) {
        msg_free(m);
        return ORC_OK;
    }
    if (hit && f->kind == ORC_FAULT_MISROUTE) dst = mod(dst + 1, nt->n);

    if (nt->trace) {
        orc_trace* t = nt->trace;
        if (t->log && t->log_len < t->log_cap) {
            orc_msg_rec* r = &t->log[t->log_len];
            r->phase = m->phase;
            r->step = m->step;
            r->src = m->src;
            r->dst = dst;
            r->chunk = m->chunk;
            r->chunk_hi = m->chunk_hi;
            r->elems = m->elems;
        }
        t->log_len++;
        if (t->sent_elems) t->sent_elems[m->src] += m->elems;
        if (t->recv_elems) t->recv_elems[dst] += m->elems;
    }
    inbox_push(&nt->boxes[dst], m);

    if (hit && f->kind == ORC_FAULT_DUP) {
        msg* d = (msg*)calloc(1, sizeof(msg));
        if (!d) return ORC_E_NOMEM;
        *d = *m;
        d->payload = (unsigned char*)malloc(m->elems ? m->elems * nt->esz : 1);
        if (!d->payload) {
            free(d);
            return ORC_E_NOMEM;
        }
        memcpy(d->payload, m->payload, m->elems * nt->esz);
        inbox_push(&nt->boxes[dst], d);
    }
    return ORC_OK;
}

/* Post a message from `src` to its ring successor. */
static int post(net* nt, msg* m) { return post_to(nt, m, mod(m->src + 1, nt->n)); }

/* Receive the next message of rank r and check its tag. */
static int receive(net* nt, int r, int phase, int step, int want_chunk, msg** out)
{
    msg* m = inbox_pop(&nt->boxes[r]);
    *out = NULL;
    if (!m) return ORC_E_EMPTY;
    if (m->src != mod(r - 1, nt->n) || m->phase != phase || m->step != step ||
        m->chunk != want_chunk) {
        msg_free(m);
        return ORC_E_TAG;
    }
    *out = m;
    return ORC_OK;
}

static int drain_check(net* nt)
{
    int rc = ORC_OK;
    for (int r = 0; r < nt->n; r++) {
        msg* m;
        while ((m = inbox_pop(&nt->boxes[r])) != NULL) {
            msg_free(m);
            rc = ORC_E_LEFTOVER;
        }
    }
    return rc;
}

/* ------------------------------------------------------------------ */
/* The ring phases                                                     */
/* ------------------------------------------------------------------ */

/* Reduce-scatter phase [RS][RING], steps 0..rs_steps-1 (normally N-1).
 * At step s rank r sends its chunk (r - s) to rank r+1 and receives chunk
 * (r - 1 - s) from rank r-1, which it adds into its own copy. */
static int phase_reduce_scatter(net* nt, unsigned char** buf, const geom* g, int rs_steps)
{
    int n = nt->n;
    for (int s = 0; s < rs_steps; s++) {
        for (int r = 0; r < n; r++) {
            int c = mod(r - s, n);
            const orc_fault* f = nt->fault;
            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_RS &&
                f->step == s && f->rank == r)
                c = mod(c + 1, n);
            msg* m = msg_make(nt, r, ORC_PHASE_RS, s, c, buf[r], chunk_len(g, c), g, 0);
            if (!m) return ORC_E_NOMEM;
            int rc = post(nt, m);
            if (rc) return rc;
        }
        for (int r = 0; r < n; r++) {
            int c = mod(r - 1 - s, n);
            msg* m;
            int rc = receive(nt, r, ORC_PHASE_RS, s, c, &m);
            if (rc) return rc;
            if (m->elems != chunk_len(g, c)) {
                msg_free(m);
                return ORC_E_TAG;
            }
            for (uint64_t k = 0; k < m->elems; k++) {
                unsigned char* mine = buf[r] + chunk_elem(g, c, k) * nt->esz;
                elem_add(nt->dt, mine, mine, m->payload + k * nt->esz);
            }
            msg_free(m);
        }
    }
    return ORC_OK;
}

/* All-gather phase of the all-reduce [RING], steps 0..ag_steps-1.  After
 * the reduce-scatter rank r owns the complete chunk r+1.  At step s rank r
 * sends chunk (r + 1 - s) and receives chunk (r - s), which overwrites its
 * copy. */
static int phase_all_gather_chunks(net* nt, unsigned char** buf, const geom* g, int ag_steps)
{
    int n = nt->n;
    for (int s = 0; s < ag_steps; s++) {
        for (int r = 0; r < n; r++) {
            int c = mod(r + 1 - s, n);
            const orc_fault* f = nt->fault;
            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_AG &&
                f->step == s && f->rank == r)
                c = mod(c + 1, n);
            msg* m = msg_make(nt, r, ORC_PHASE_AG, s, c, buf[r], chunk_len(g, c), g, 0);
            if (!m) return ORC_E_NOMEM;
            int rc = post(nt, m);
            if (rc) return rc;
        }
        for (int r = 0; r < n; r++) {
            int c = mod(r - s, n);
            msg* m;
            int rc = receive(nt, r, ORC_PHASE_AG, s, c, &m);
            if (rc) return rc;
            if (m->elems != chunk_len(g, c)) {
                msg_free(m);
                return ORC_E_TAG;
            }
            for (uint64_t k = 0; k < m->elems; k++)
                memcpy(buf[r] + chunk_elem(g, c, k) * nt->esz, m->payload + k * nt->esz, nt->esz);
            msg_free(m);
        }
    }
    return ORC_OK;
}

static int check_dtype_n(int dt, int n)
{
    if (elem_size(dt) == 0) return ORC_E_ARG;
    if (n < 1) return ORC_E_ARG;
    return ORC_OK;
}

static net* net_new(int dt, int n, orc_trace* trace, const orc_fault* fault)
{
    net* nt = (net*)calloc(1, sizeof(net));
    if (!nt) return NULL;
    nt->boxes = (inbox*)calloc((size_t)n, sizeof(inbox));
    if (!nt->boxes) {
        free(nt);
        return NULL;
    }
    nt->dt = dt;
    nt->n = n;
    nt->esz = elem_size(dt);
    nt->trace = trace;
    nt->fault = fault;
    if (trace) {
        trace->log_len = 0;
        for (int r = 0; r < n; r++) {
            if (trace->sent_elems) trace->sent_elems[r] = 0;
            if (trace->recv_elems) trace->recv_elems[r] = 0;
        }
    }
    return nt;
}

static void net_free(net* nt)
{
    if (!nt) return;
    drain_check(nt);
    free(nt->boxes);
    free(nt);
}

static unsigned char** rank_state_new(int n, uint64_t elems, size_t esz)
{
    unsigned char** buf = (unsigned char**)calloc((size_t)n, sizeof(unsigned char*));
    if (!buf) return NULL;
    for (int r = 0; r < n; r++) {
        buf[r] = (unsigned char*)malloc(elems ? elems * esz : 1);
        if (!buf[r]) {
            for (int q = 0; q < r; q++) free(buf[q]);
            free(buf);
            return NULL;
        }
    }
    return buf;
}

static void rank_state_free(unsigned char** buf, int n)
{
    if (!buf) return;
    for (int r = 0; r < n; r++) free(buf[r]);
    free(buf);
}

/* ------------------------------------------------------------------ */
/* Exported: literal ring simulations                                  */
/* ------------------------------------------------------------------ */

/* Ring all-reduce: reduce-scatter then all-gather over the flat chunking.
 * x[r], y[r]: count elements each.  rs_steps / ag_steps < 0 mean N-1
 * (smaller values stop the simulation early so tests can inspect the
 * intermediate rank buffers, which are then written to y). */
int orc_ring_allreduce_steps(int dt, int n, uint64_t count, const void* const* x, void* const* y,
                             int rs_steps, int ag_steps, orc_trace* trace, const orc_fault* fault)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (rs_steps < 0) rs_steps = n - 1;
    if (ag_steps < 0) ag_steps = n - 1;
    if (rs_steps > n - 1 || ag_steps > n - 1) return ORC_E_ARG;
    geom g = {count, 1, count, n};
    size_t esz = elem_size(dt);
    unsigned char** buf = rank_state_new(n, count, esz);
    if (!buf) return ORC_E_NOMEM;
    for (int r = 0; r < n; r++) memcpy(buf[r], x[r], count * esz);
    net* nt = net_new(dt, n, trace, fault);
    if (!nt) {
        rank_state_free(buf, n);
        return ORC_E_NOMEM;
    }
    rc = phase_reduce_scatter(nt, buf, &g, rs_steps);
    if (!rc) rc = phase_all_gather_chunks(nt, buf, &g, ag_steps);
    if (!rc) rc = drain_check(nt);
    if (!rc)
        for (int r = 0; r < n; r++) memcpy(y[r], buf[r], count * esz);
    net_free(nt);
    rank_state_free(buf, n);
    return rc;
}

int orc_ring_allreduce(int dt, int n, uint64_t count, const void* const* x, void* const* y)
{
    return orc_ring_allreduce_steps(dt, n, count, x, y, -1, -1, NULL, NULL);
}

/* Ring reduce-scatter.  Each rank's input is [outer, count/outer]; the
 * output of rank c is the reduced chunk c (chunk_len elements, laid out
 * [outer, w] when outer > 1).  The reduce-scatter phase leaves the
 * complete chunk c at rank c-1, from where it is delivered unchanged. */
int orc_ring_reduce_scatter(int dt, int n, uint64_t count, uint64_t outer, const void* const* x,
                            void* const* y, orc_trace* trace, const orc_fault* fault)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (outer == 0 || count % outer != 0) return ORC_E_ARG;
    geom g = {count, outer, count / outer, n};
    if (outer > 1 && g.row % (uint64_t)n != 0) return ORC_E_ARG;
    size_t esz = elem_size(dt);
    unsigned char** buf = rank_state_new(n, count, esz);
    if (!buf) return ORC_E_NOMEM;
    for (int r = 0; r < n; r++) memcpy(buf[r], x[r], count * esz);
    net* nt = net_new(dt, n, trace, fault);
    if (!nt) {
        rank_state_free(buf, n);
        return ORC_E_NOMEM;
    }
    rc = phase_reduce_scatter(nt, buf, &g, n - 1);
    if (!rc) rc = drain_check(nt);
    if (!rc) {
        for (int c = 0; c < n; c++) {
            int holder = mod(c - 1, n);
            unsigned char* out = (unsigned char*)y[c];
            for (uint64_t k = 0; k < chunk_len(&g, c); k++)
                memcpy(out + k * esz, buf[holder] + chunk_elem(&g, c, k) * esz, esz);
        }
    }
    net_free(nt);
    rank_state_free(buf, n);
    return rc;
}

/* Ring all-gather.  Each rank's input is [outer, row] (row = count/outer);
 * each output is [outer, n*row] with rank q's input in column slab q.
 * Rank r starts with its own slab; at step s it sends slab (r - s) to
 * rank r+1 and receives slab (r - 1 - s) from rank r-1. */
int orc_ring_all_gather(int dt, int n, uint64_t count, uint64_t outer, const void* const* x,
                        void* const* y, orc_trace* trace, const orc_fault* fault)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (outer == 0 || count % outer != 0) return ORC_E_ARG;
    geom g = {count, outer, count / outer, n};
    size_t esz = elem_size(dt);
    uint64_t out_elems = count * (uint64_t)n;
    unsigned char** buf = rank_state_new(n, out_elems, esz);
    if (!buf) return ORC_E_NOMEM;
    for (int r = 0; r < n; r++) {
        memset(buf[r], 0, out_elems * esz);
        const unsigned char* in = (const unsigned char*)x[r];
        for (uint64_t k = 0; k < count; k++) {
            uint64_t o = k / g.row, j = k % g.row;
            memcpy(buf[r] + (o * g.row * (uint64_t)n + (uint64_t)r * g.row + j) * esz, in + k * esz, esz);
        }
    }
    net* nt = net_new(dt, n, trace, fault);
    if (!nt) {
        rank_state_free(buf, n);
        return ORC_E_NOMEM;
    }
    for (int s = 0; s < n - 1 && !rc; s++) {
        for (int r = 0; r < n && !rc; r++) {
            int slab = mod(r - s, n);
            const orc_fault* f = fault;
            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_AG &&
                f->step == s && f->rank == r)
                slab = mod(slab + 1, n);
            msg* m = msg_make(nt, r, ORC_PHASE_AG, s, slab, buf[r], count, &g, 1);
            if (!m) rc = ORC_E_NOMEM;
            else rc = post(nt, m);
        }
        for (int r = 0; r < n && !rc; r++) {
            int slab = mod(r - 1 - s, n);
            msg* m;
            rc = receive(nt, r, ORC_PHASE_AG, s, slab, &m);
            if (rc) break;
            for (uint64_t k = 0; k < m->elems; k++) {
                uint64_t o = k / g.row, j = k % g.row;
                memcpy(buf[r] + (o * g.row * (uint64_t)n + (uint64_t)slab * g.row + j) * esz,
                       m->payload + k * esz, esz);
            }
            msg_free(m);
        }
    }
    if (!rc) rc = drain_check(nt);
    if (!rc)
        for (int r = 0; r < n; r++) memcpy(y[r], buf[r], out_elems * esz);
    net_free(nt);
    rank_state_free(buf, n);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Exported: the fused (naive) reductions [NAIVE]                      */
/* ------------------------------------------------------------------ */

/* y[r][i] = round(x[0][i] + x[1][i] + ... + x[n-1][i]), folded left in
 * rank order in the accumulator, rounded once; the same value for all r. */
int orc_fused_allreduce(int dt, int n, uint64_t count, const void* const* x, void* const* y)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    size_t esz = elem_size(dt);
    for (uint64_t i = 0; i < count; i++) {
        acc_t acc;
        acc_set(dt, &acc, (const unsigned char*)x[0] + i * esz);
        for (int r = 1; r < n; r++) acc_add(dt, &acc, (const unsigned char*)x[r] + i * esz);
        for (int r = 0; r < n; r++) acc_store(dt, &acc, (unsigned char*)y[r] + i * esz);
    }
    return ORC_OK;
}

/* Fused reduce-scatter: y[c][k] = the rank-order fold of element k of
 * chunk c over all ranks, rounded once. */
int orc_fused_reduce_scatter(int dt, int n, uint64_t count, uint64_t outer, const void* const* x,
                             void* const* y)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (outer == 0 || count % outer != 0) return ORC_E_ARG;
    geom g = {count, outer, count / outer, n};
    if (outer > 1 && g.row % (uint64_t)n != 0) return ORC_E_ARG;
    size_t esz = elem_size(dt);
    for (int c = 0; c < n; c++) {
        for (uint64_t k = 0; k < chunk_len(&g, c); k++) {
            uint64_t at = chunk_elem(&g, c, k);
            acc_t acc;
            acc_set(dt, &acc, (const unsigned char*)x[0] + at * esz);
            for (int r = 1; r < n; r++) acc_add(dt, &acc, (const unsigned char*)x[r] + at * esz);
            acc_store(dt, &acc, (unsigned char*)y[c] + k * esz);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Exported: per-element closed forms (for sampled checks at full size) */
/* ------------------------------------------------------------------ */

/* Ring all-reduce result at flat index idx[k]: chunk c = chunk_of(idx)
 * travels c -> c+1 -> ... -> c+N-1 during the reduce-scatter, so its value
 * is ((x_c (+) x_{c+1}) (+) x_{c+2}) ... (+) x_{c+N-1}, every (+) in storage
 * semantics. */
int orc_ring_allreduce_at(int dt, int n, uint64_t count, const void* const* x, const uint64_t* idx,
                          uint64_t m, void* out)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    size_t esz = elem_size(dt);
    unsigned char partial[8];
    for (uint64_t k = 0; k < m; k++) {
        uint64_t i = idx[k];
        if (i >= count) return ORC_E_ARG;
        int c = chunk_of(count, n, i);
        memcpy(partial, (const unsigned char*)x[c] + i * esz, esz);
        for (int t = 1; t < n; t++) {
            int r = mod(c + t, n);
            elem_add(dt, partial, partial, (const unsigned char*)x[r] + i * esz);
        }
        memcpy((unsigned char*)out + k * esz, partial, esz);
    }
    return ORC_OK;
}

/* Fused all-reduce result at flat index idx[k] (rank-order fold). */
int orc_fused_allreduce_at(int dt, int n, uint64_t count, const void* const* x, const uint64_t* idx,
                           uint64_t m, void* out)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    size_t esz = elem_size(dt);
    for (uint64_t k = 0; k < m; k++) {
        uint64_t i = idx[k];
        if (i >= count) return ORC_E_ARG;
        acc_t acc;
        acc_set(dt, &acc, (const unsigned char*)x[0] + i * esz);
        for (int r = 1; r < n; r++) acc_add(dt, &acc, (const unsigned char*)x[r] + i * esz);
        acc_store(dt, &acc, (unsigned char*)out + k * esz);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Halving-doubling [HD]                                               */
/* ------------------------------------------------------------------ */

static int is_pow2(int n) { return n >= 1 && (n & (n - 1)) == 0; }

/* Elements in the block range [lo, hi). */
static uint64_t range_len(const geom* g, int lo, int hi)
{
    uint64_t total = 0;
    for (int b = lo; b < hi; b++) total += chunk_len(g, b);
    return total;
}

/* Flat index of the k-th element of the block range [lo, hi), taking the
 * blocks in order and each block's elements in order. */
static uint64_t range_elem(const geom* g, int lo, int hi, uint64_t k)
{
    for (int b = lo; b < hi; b++) {
        uint64_t len = chunk_len(g, b);
        if (k < len) return chunk_elem(g, b, k);
        k -= len;
    }
    return 0; /* not reached for k < range_len */
}

/* Flat index, in an [outer, n*row] all-gather output, of the k-th element
 * of the slab range [lo, hi) (row by row, slab by slab). */
static uint64_t slab_range_elem(const geom* g, int lo, int hi, uint64_t k)
{
    uint64_t width = (uint64_t)(hi - lo) * g->row;
    uint64_t o = k / width, rem = k % width;
    uint64_t q = (uint64_t)lo + rem / g->row, j = rem % g->row;
    return o * g->row * (uint64_t)g->n + q * g->row + j;
}

static msg* range_msg(const net* nt, int src, int phase, int step, int lo, int hi, const unsigned char* buf,
                      const geom* g, int slabs)
{
    uint64_t elems = slabs ? (uint64_t)(hi - lo) * g->count : range_len(g, lo, hi);
    msg* m = (msg*)calloc(1, sizeof(msg));
    if (!m) return NULL;
    m->payload = (unsigned char*)malloc(elems ? elems * nt->esz : 1);
    if (!m->payload) {
        free(m);
        return NULL;
    }
    m->src = src;
    m->phase = phase;
    m->step = step;
    m->chunk = lo;
    m->chunk_hi = hi;
    m->elems = elems;
    for (uint64_t k = 0; k < elems; k++) {
        uint64_t at = slabs ? slab_range_elem(g, lo, hi, k) : range_elem(g, lo, hi, k);
        memcpy(m->payload + k * nt->esz, buf + at * nt->esz, nt->esz);
    }
    return m;
}

/* Receive rank r's next message and check it came from `src` with the
 * expected phase, step and block range. */
static int receive_range(net* nt, int r, int src, int phase, int step, int lo, int hi, msg** out)
{
    msg* m = inbox_pop(&nt->boxes[r]);
    *out = NULL;
    if (!m) return ORC_E_EMPTY;
    if (m->src != src || m->phase != phase || m->step != step || m->chunk != lo || m->chunk_hi != hi) {
        msg_free(m);
        return ORC_E_TAG;
    }
    *out = m;
    return ORC_OK;
}

/* Recursive halving.  lo[r], hi[r]: rank r's current block range (start
 * [0, N)).  At the step with distance d the range is split in two; the rank
 * whose bit d is clear keeps the lower half, its partner r XOR d the upper
 * half; each sends the other half to the partner and adds the half it
 * receives into its own copy.  After log2 N steps rank r holds block r. */
static int phase_halving(net* nt, unsigned char** buf, const geom* g, int* lo, int* hi, int steps)
{
    int n = nt->n, step = 0;
    for (int d = n / 2; d >= 1 && step < steps; d /= 2, step++) {
        for (int r = 0; r < n; r++) {
            int mid = (lo[r] + hi[r]) / 2;
            int upper = (r & d) != 0;
            int give_lo = upper ? lo[r] : mid, give_hi = upper ? mid : hi[r];
            const orc_fault* f = nt->fault;
            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_HD_RS && f->step == step &&
                f->rank == r) {
                give_lo = upper ? mid : lo[r];
                give_hi = upper ? hi[r] : mid;
            }
            msg* m = range_msg(nt, r, ORC_PHASE_HD_RS, step, give_lo, give_hi, buf[r], g, 0);
            if (!m) return ORC_E_NOMEM;
            int rc = post_to(nt, m, r ^ d);
            if (rc) return rc;
        }
        for (int r = 0; r < n; r++) {
            int mid = (lo[r] + hi[r]) / 2;
            int upper = (r & d) != 0;
            int keep_lo = upper ? mid : lo[r], keep_hi = upper ? hi[r] : mid;
            msg* m;
            int rc = receive_range(nt, r, r ^ d, ORC_PHASE_HD_RS, step, keep_lo, keep_hi, &m);
            if (rc) return rc;
            for (uint64_t k = 0; k < m->elems; k++) {
                unsigned char* mine = buf[r] + range_elem(g, keep_lo, keep_hi, k) * nt->esz;
                elem_add(nt->dt, mine, m->payload + k * nt->esz, mine);
            }
            msg_free(m);
            lo[r] = keep_lo;
            hi[r] = keep_hi;
        }
    }
    return ORC_OK;
}

/* Recursive doubling.  At the step with distance d (1, 2, ..., N/2) rank r
 * sends its whole current range to r XOR d and copies the partner's range
 * into its own buffer; the two ranges are adjacent and merge.  `slabs`
 * selects all-gather slabs of an [outer, N*row] buffer instead of blocks. */
static int phase_doubling(net* nt, unsigned char** buf, const geom* g, int* lo, int* hi, int steps, int slabs)
{
    int n = nt->n, step = 0;
    int plo[64], phi[64];
    for (int d = 1; d < n && step < steps; d *= 2, step++) {
        for (int r = 0; r < n; r++) {
            int give_lo = lo[r], give_hi = hi[r];
            const orc_fault* f = nt->fault;
            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_HD_AG && f->step == step &&
                f->rank == r) {
                give_lo = lo[r ^ d];
                give_hi = hi[r ^ d];
            }
            msg* m = range_msg(nt, r, ORC_PHASE_HD_AG, step, give_lo, give_hi, buf[r], g, slabs);
            if (!m) return ORC_E_NOMEM;
            int rc = post_to(nt, m, r ^ d);
            if (rc) return rc;
        }
        for (int r = 0; r < n; r++) {
            plo[r] = lo[r];
            phi[r] = hi[r];
        }
        for (int r = 0; r < n; r++) {
            int p = r ^ d;
            msg* m;
            int rc = receive_range(nt, r, p, ORC_PHASE_HD_AG, step, plo[p], phi[p], &m);
            if (rc) return rc;
            for (uint64_t k = 0; k < m->elems; k++) {
                uint64_t at = slabs ? slab_range_elem(g, plo[p], phi[p], k) : range_elem(g, plo[p], phi[p], k);
                memcpy(buf[r] + at * nt->esz, m->payload + k * nt->esz, nt->esz);
            }
            msg_free(m);
            lo[r] = plo[r] < plo[p] ? plo[r] : plo[p];
            hi[r] = phi[r] > phi[p] ? phi[r] : phi[p];
        }
    }
    return ORC_OK;
}

static int log2i(int n)
{
    int k = 0;
    while ((1 << k) < n) k++;
    return k;
}

/* Halving-doubling all-reduce (N a power of two, at most 64).  rs_steps /
 * ag_steps < 0 mean log2 N; smaller values stop early so tests can inspect
 * the intermediate rank buffers. */
int orc_hd_allreduce_steps(int dt, int n, uint64_t count, const void* const* x, void* const* y, int rs_steps,
                           int ag_steps, orc_trace* trace, const orc_fault* fault)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (!is_pow2(n) || n > 64) return ORC_E_ARG;
    int k = log2i(n);
    if (rs_steps < 0) rs_steps = k;
    if (ag_steps < 0) ag_steps = k;
    if (rs_steps > k || ag_steps > k) return ORC_E_ARG;
    geom g = {count, 1, count, n};
    size_t esz = elem_size(dt);
    unsigned char** buf = rank_state_new(n, count, esz);
    if (!buf) return ORC_E_NOMEM;
    for (int r = 0; r < n; r++) memcpy(buf[r], x[r], count * esz);
    net* nt = net_new(dt, n, trace, fault);
    if (!nt) {
        rank_state_free(buf, n);
        return ORC_E_NOMEM;
    }
    int lo[64], hi[64];
    for (int r = 0; r < n; r++) {
        lo[r] = 0;
        hi[r] = n;
    }
    rc = phase_halving(nt, buf, &g, lo, hi, rs_steps);
    if (!rc && rs_steps == k) rc = phase_doubling(nt, buf, &g, lo, hi, ag_steps, 0);
    if (!rc) rc = drain_check(nt);
    if (!rc)
        for (int r = 0; r < n; r++) memcpy(y[r], buf[r], count * esz);
    net_free(nt);
    rank_state_free(buf, n);
    return rc;
}

/* Halving-doubling reduce-scatter: recursive halving, after which rank c
 * holds block c, delivered unchanged as output c. */
int orc_hd_reduce_scatter(int dt, int n, uint64_t count, uint64_t outer, const void* const* x, void* const* y,
                          orc_trace* trace, const orc_fault* fault)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (!is_pow2(n) || n > 64) return ORC_E_ARG;
    if (outer == 0 || count % outer != 0) return ORC_E_ARG;
    geom g = {count, outer, count / outer, n};
    if (outer > 1 && g.row % (uint64_t)n != 0) return ORC_E_ARG;
    size_t esz = elem_size(dt);
    unsigned char** buf = rank_state_new(n, count, esz);
    if (!buf) return ORC_E_NOMEM;
    for (int r = 0; r < n; r++) memcpy(buf[r], x[r], count * esz);
    net* nt = net_new(dt, n, trace, fault);
    if (!nt) {
        rank_state_free(buf, n);
        return ORC_E_NOMEM;
    }
    int lo[64], hi[64];
    for (int r = 0; r < n; r++) {
        lo[r] = 0;
        hi[r] = n;
    }
    rc = phase_halving(nt, buf, &g, lo, hi, log2i(n));
    if (!rc) rc = drain_check(nt);
    if (!rc) {
        for (int c = 0; c < n; c++) {
            if (lo[c] != c || hi[c] != c + 1) {
                rc = ORC_E_TAG;
                break;
            }
            unsigned char* out = (unsigned char*)y[c];
            for (uint64_t k = 0; k < chunk_len(&g, c); k++)
                memcpy(out + k * esz, buf[c] + chunk_elem(&g, c, k) * esz, esz);
        }
    }
    net_free(nt);
    rank_state_free(buf, n);
    return rc;
}

/* Halving-doubling all-gather: recursive doubling over the slabs of the
 * [outer, N*row] outputs, starting from each rank's own slab. */
int orc_hd_all_gather(int dt, int n, uint64_t count, uint64_t outer, const void* const* x, void* const* y,
                      orc_trace* trace, const orc_fault* fault)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (!is_pow2(n) || n > 64) return ORC_E_ARG;
    if (outer == 0 || count % outer != 0) return ORC_E_ARG;
    geom g = {count, outer, count / outer, n};
    size_t esz = elem_size(dt);
    uint64_t out_elems = count * (uint64_t)n;
    unsigned char** buf = rank_state_new(n, out_elems, esz);
    if (!buf) return ORC_E_NOMEM;
    int lo[64], hi[64];
    for (int r = 0; r < n; r++) {
        memset(buf[r], 0, out_elems * esz);
        for (uint64_t k = 0; k < count; k++)
            memcpy(buf[r] + slab_range_elem(&g, r, r + 1, k) * esz, (const unsigned char*)x[r] + k * esz, esz);
        lo[r] = r;
        hi[r] = r + 1;
    }
    net* nt = net_new(dt, n, trace, fault);
    if (!nt) {
        rank_state_free(buf, n);
        return ORC_E_NOMEM;
    }
    rc = phase_doubling(nt, buf, &g, lo, hi, log2i(n), 1);
    if (!rc) rc = drain_check(nt);
    if (!rc)
        for (int r = 0; r < n; r++) memcpy(y[r], buf[r], out_elems * esz);
    net_free(nt);
    rank_state_free(buf, n);
    return rc;
}

/* ------------------------------------------------------------------ */
/* Binomial-tree all-gather [TREE]                                     */
/* ------------------------------------------------------------------ */

/* Gather to rank 0.  hi[r]: rank r holds slabs [r, hi[r]) (its own slab to
 * begin with).  At the step with distance d (1, 2, 4, ... while d < N) rank
 * r with r mod 2d == d sends [r, hi[r]) to rank r - d, which copies the
 * slabs into its buffer; ranks r with r mod 2d == 0 and r + d < N receive.
 * After ceil(log2 N) steps rank 0 holds all N slabs. */
static int phase_tree_gather(net* nt, unsigned char** buf, const geom* g, int* hi)
{
    int n = nt->n, step = 0;
    for (int d = 1; d < n; d *= 2, step++) {
        for (int r = 0; r < n; r++) {
            if (r % (2 * d) != d) continue;
            int lo = r, top = hi[r];
            const orc_fault* f = nt->fault;
            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_TREE_GATHER && f->step == step &&
                f->rank == r) {
                lo -= d; /* the receiver's own slabs instead */
                top -= d;
            }
            msg* m = range_msg(nt, r, ORC_PHASE_TREE_GATHER, step, lo, top, buf[r], g, 1);
            if (!m) return ORC_E_NOMEM;
            int rc = post_to(nt, m, r - d);
            if (rc) return rc;
        }
        for (int r = 0; r < n; r++) {
            if (r % (2 * d) != 0 || r + d >= n) continue;
            int p = r + d;
            msg* m;
            int rc = receive_range(nt, r, p, ORC_PHASE_TREE_GATHER, step, p, hi[p], &m);
            if (rc) return rc;
            for (uint64_t k = 0; k < m->elems; k++)
                memcpy(buf[r] + slab_range_elem(g, p, hi[p], k) * nt->esz, m->payload + k * nt->esz, nt->esz);
            msg_free(m);
            hi[r] = hi[p];
        }
    }
    return ORC_OK;
}

/* Broadcast from rank 0 along the same tree in reverse: at the step with
 * distance d (the largest power of two below N, then d/2, ..., 1) rank r
 * with r mod 2d == 0 and r + d < N sends all N slabs to rank r + d, which
 * copies them into its buffer. */
static int phase_tree_bcast(net* nt, unsigned char** buf, const geom* g)
{
    int n = nt->n, step = 0, top = 1;
    while (2 * top < n) top *= 2;
    for (int d = top; n > 1 && d >= 1; d /= 2, step++) {
        for (int r = 0; r < n; r++) {
            if (r % (2 * d) != 0 || r + d >= n) continue;
            int top_slab = n;
            const orc_fault* f = nt->fault;
            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_TREE_BCAST && f->step == step &&
                f->rank == r)
                top_slab = n - 1; /* all but the last slab */
            msg* m = range_msg(nt, r, ORC_PHASE_TREE_BCAST, step, 0, top_slab, buf[r], g, 1);
            if (!m) return ORC_E_NOMEM;
            int rc = post_to(nt, m, r + d);
            if (rc) return rc;
        }
        for (int r = 0; r < n; r++) {
            if (r % (2 * d) != d) continue;
            msg* m;
            int rc = receive_range(nt, r, r - d, ORC_PHASE_TREE_BCAST, step, 0, n, &m);
            if (rc) return rc;
            for (uint64_t k = 0; k < m->elems; k++)
                memcpy(buf[r] + slab_range_elem(g, 0, n, k) * nt->esz, m->payload + k * nt->esz, nt->esz);
            msg_free(m);
        }
    }
    return ORC_OK;
}

/* Tree all-gather over the slabs of [outer, N*row] outputs: every rank
 * starts with its own slab, the gather collects all slabs at rank 0, the
 * broadcast hands rank 0's buffer to every rank.  Any N from 1 to 64. */
int orc_tree_all_gather(int dt, int n, uint64_t count, uint64_t outer, const void* const* x, void* const* y,
                        orc_trace* trace, const orc_fault* fault)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (n > 64) return ORC_E_ARG;
    if (outer == 0 || count % outer != 0) return ORC_E_ARG;
    geom g = {count, outer, count / outer, n};
    size_t esz = elem_size(dt);
    uint64_t out_elems = count * (uint64_t)n;
    unsigned char** buf = rank_state_new(n, out_elems, esz);
    if (!buf) return ORC_E_NOMEM;
    int hi[64];
    for (int r = 0; r < n; r++) {
        memset(buf[r], 0, out_elems * esz);
        for (uint64_t k = 0; k < count; k++)
            memcpy(buf[r] + slab_range_elem(&g, r, r + 1, k) * esz, (const unsigned char*)x[r] + k * esz, esz);
        hi[r] = r + 1;
    }
    net* nt = net_new(dt, n, trace, fault);
    if (!nt) {
        rank_state_free(buf, n);
        return ORC_E_NOMEM;
    }
    rc = phase_tree_gather(nt, buf, &g, hi);
    if (!rc && hi[0] != n) rc = ORC_E_TAG;
    if (!rc) rc = phase_tree_bcast(nt, buf, &g);
    if (!rc) rc = drain_check(nt);
    if (!rc)
        for (int r = 0; r < n; r++) memcpy(y[r], buf[r], out_elems * esz);
    net_free(nt);
    rank_state_free(buf, n);
    return rc;
}

/* Halving-doubling result at flat index idx[k].  Every rank and every block
 * gets the same butterfly: pairs at distance N/2 first, then pairs of pairs
 * at distance N/4, and so on, each partial rounded to the storage type:
 * v[r] = x_r[i]; for d = N/2 .. 1: v[r] = v[r] (+) v[r + d] for r < d;
 * the result is v[0]. */
int orc_hd_allreduce_at(int dt, int n, uint64_t count, const void* const* x, const uint64_t* idx, uint64_t m,
                        void* out)
{
    int rc = check_dtype_n(dt, n);
    if (rc) return rc;
    if (!is_pow2(n) || n > 64) return ORC_E_ARG;
    size_t esz = elem_size(dt);
    unsigned char v[64 * 8];
    for (uint64_t k = 0; k < m; k++) {
        uint64_t i = idx[k];
        if (i >= count) return ORC_E_ARG;
        for (int r = 0; r < n; r++) memcpy(v + r * esz, (const unsigned char*)x[r] + i * esz, esz);
        for (int d = n / 2; d >= 1; d /= 2)
            for (int r = 0; r < d; r++) elem_add(dt, v + r * esz, v + r * esz, v + (r + d) * esz);
        memcpy((unsigned char*)out + k * esz, v, esz);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Exported: codecs and partition, for the oracle's own pins           */
/* ------------------------------------------------------------------ */

void orc_f32_to_f16(const float* in, uint16_t* out, uint64_t m)
{
    for (uint64_t k = 0; k < m; k++) out[k] = f16_encode(in[k]);
}
void orc_f16_to_f32(const uint16_t* in, float* out, uint64_t m)
{
    for (uint64_t k = 0; k < m; k++) out[k] = f16_decode(in[k]);
}
void orc_f32_to_bf16(const float* in, uint16_t* out, uint64_t m)
{
    for (uint64_t k = 0; k < m; k++) out[k] = bf16_encode(in[k]);
}
void orc_bf16_to_f32(const uint16_t* in, float* out, uint64_t m)
{
    for (uint64_t k = 0; k < m; k++) out[k] = bf16_decode(in[k]);
}

/* Storage-semantics add of two element arrays (for codec/arith pins). */
int orc_add(int dt, const void* a, const void* b, void* out, uint64_t m)
{
    size_t esz = elem_size(dt);
    if (!esz) return ORC_E_ARG;
    for (uint64_t k = 0; k < m; k++)
        elem_add(dt, (unsigned char*)out + k * esz, (const unsigned char*)a + k * esz,
                 (const unsigned char*)b + k * esz);
    return ORC_OK;
}

/* Offset and length of chunk c of a flat buffer of `count` elements. */
int orc_chunk_range(uint64_t count, int n, int c, uint64_t* off, uint64_t* len)
{
    if (n < 1 || c < 0 || c >= n) return ORC_E_ARG;
    geom g = {count, 1, count, n};
    *len = chunk_len(&g, c);
    *off = (uint64_t)c * (count / (uint64_t)n);
    return ORC_OK;
}
