// la_api.hip -- the C ABI of liblinattn (declared in include/la.h): argument validation,
// kernel selection, sequence split and per-stream scratch memory.
#include "la.h"
#include "la_launch.h"

#include <mutex>
#include <stdint.h>
#include <vector>

namespace {

constexpr int LA_VERSION = (0 << 16) | (1 << 8) | 0;

enum Form { CAUSAL = 0, GLOBAL = 1, DECODE = 2 };

// Target number of workgroups per launch on an MI355X (256 CUs). The d = 128 matrix-core
// kernels get one wave of 256 workgroups: the causal kernel holds a whole CU (its LDS), and the
// segment sums, though two fit per CU, stream faster one per CU (measured on MI355X for the
// global form B=1 H=8 N=100000: 63 segments per head, two per CU, 200.6 us per call; 32
// segments, one per CU, 195.5 us). The other kernels fit two per CU. More segments than that
// only add segment-state traffic (66 KB read and written per extra segment at d = 128).
constexpr long kCUs = 256;
constexpr long kMinChunks = 4;

bool dim_ok(int x) { return x == 16 || x == 32 || x == 64 || x == 128; }

constexpr int kRfMaxFeatures = 4096; // projections per random-feature map
constexpr size_t kLdsBytes = 160 * 1024; // LDS one workgroup can hold on gfx950

struct Span {
    uintptr_t lo, hi; // [lo, hi); empty when lo == hi
};

Span span(const void *p, size_t bytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return p ? Span{a, a + bytes} : Span{0, 0};
}

bool overlap(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
    bool mfma;  // bf16 matrix-core family
    bool mfma32; // float32 matrix-core family
    bool shortseq; // causal, one segment of at most 64 tokens: the one-chunk kernel (no decay)
    int chunk;  // tokens per chunk
    int L;      // tokens per segment
    int P;      // segments per head
    long BH;
    size_t ws_bytes;
};

// Shape/size checks and the launch plan (no pointer checks). Returns LA_OK or a status.
int make_plan(Form form, int B, int H, int N, int d, int dv, int chunk, int seg_len, int dtype,
              Plan *plan)
{
    if (dtype != LA_F32 && dtype != LA_BF16)
        return LA_EINVAL;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || dv <= 0 || chunk < 0 || seg_len < 0)
        return LA_EINVAL;
    if (form == DECODE && N != 1)
        return LA_EINVAL;
    if (!dim_ok(d) || !dim_ok(dv))
        return LA_ENOTSUP;
    const size_t BH = (size_t)B * (size_t)H;
    // 32-bit grid and per-head index arithmetic
    if (BH > (size_t)INT32_MAX / 8 || (size_t)N * (size_t)(d > dv ? d : dv) > (size_t)INT32_MAX)
        return LA_ENOTSUP;

    Plan pl{};
    pl.BH = (long)BH;
    if (form == DECODE) {
        *plan = pl;
        return LA_OK;
    }
    const bool mfma_ok = dtype == LA_BF16 && d == dv && (d == 64 || d == 128);
    const bool mfma32_ok = dtype == LA_F32 && d == dv && (d == 64 || d == 128);
    if (chunk == 0) {
        pl.mfma = mfma_ok;
        pl.mfma32 = mfma32_ok;
        // the vector-ALU kernels' work within a chunk grows with its square (sums over the
        // chunk's keys per query), which dominates at their head sizes: chunk 16 for the causal
        // form, 32 for the global read, which has no such sums (measured on MI355X, causal
        // B=1 H=8 N=4096 d=32 float32 68.4 against 87.1 us, B=4 H=8 N=2048 d=16 47.3 against
        // 59.2; global B=1 H=8 N=100000 d=32 bf16 578 us at chunk 32 against 638 at 16)
        pl.chunk = mfma_ok ? 64 : mfma32_ok ? 32 : form == CAUSAL ? 16 : 32;
    } else if (chunk == 64 && mfma_ok) {
        pl.mfma = true;
        pl.chunk = 64;
    } else if (chunk == 32 && mfma32_ok) {
        pl.mfma32 = true;
        pl.chunk = 32;
    } else if (chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128) {
        // the vector-ALU kernels take any chunk whose working set fits the 160 KiB of LDS a
        // workgroup can hold (chunks 64 and 128 at small head sizes)
        if (la::valu_lds_bytes(d, dv, chunk) > kLdsBytes)
            return LA_ENOTSUP;
        pl.mfma = false;
        pl.chunk = chunk;
    } else {
        return LA_ENOTSUP;
    }

    const long nchunks = (N + pl.chunk - 1) / pl.chunk;
    if (seg_len > 0) {
        if (seg_len % pl.chunk != 0)
            return LA_ENOTSUP;
        pl.L = seg_len;
    } else {
        // one causal workgroup per CU for the bf16 kernels at d = 128 and the float32 ones
        // (their LDS holds one), two elsewhere
        const long target = ((pl.mfma && d == 128) || pl.mfma32) ? kCUs : 2 * kCUs;
        long want = (target + (long)BH - 1) / (long)BH; // segments per head
        // matrix-core kernels: at least kMinChunks chunks per segment; a segment's fixed costs
        // (its sum written and scanned, its prefix read, the pipeline filled) outweigh its
        // parallelism below that (measured on MI355X, B=4 H=8 N=2048 d=64: 16 segments of 2
        // chunks 27.1 us per call, 8 segments of 4 chunks 24.8 us, both with cold caches).
        // The vector-ALU kernels otherwise keep every segment, except that a sequence of at most
        // 64 tokens (or two chunks) runs as one segment: one launch instead of three (B=1 H=1
        // N=64 d=16 float32: 14.0 us per call at chunk 16 as one segment, 19.7 us as four,
        // 16.7 us at chunk 32; at N=128, eight segments of one chunk take 20.0 us, one 25.9 us).
        const bool matrix = pl.mfma || pl.mfma32;
        const bool short_seq = N <= (64 > 2 * pl.chunk ? 64 : 2 * pl.chunk);
        const long most = !matrix ? (short_seq ? 1 : nchunks)
                                  : nchunks / kMinChunks > 1 ? nchunks / kMinChunks : 1;
        if (want > most)
            want = most;
        pl.L = (int)((nchunks + want - 1) / want) * pl.chunk;
    }
    pl.P = (int)((N + (long)pl.L - 1) / pl.L);
    // a short sequence in one segment, chunk left to the library: the whole sequence as one
    // chunk, evaluated directly (see k_short)
    pl.shortseq = form == CAUSAL && chunk == 0 && !pl.mfma && !pl.mfma32 && pl.P == 1 &&
                  la::short_ok(N, d, dv);
    if ((size_t)pl.P * BH > (size_t)INT32_MAX / 8)
        return LA_ENOTSUP;
    const size_t E = (size_t)d * dv + d;
    pl.ws_bytes = pl.P > 1 ? BH * (size_t)pl.P * E * sizeof(float) : 0;
    *plan = pl;
    return LA_OK;
}

// Full validation of an entry point's arguments: pointers, then make_plan. S0, z0 are the
// causal form's initial state (read only; may be the same buffers as S, z, which receive the
// final state); the other forms pass S0 = z0 = NULL.
int validate(Form form, const void *q, const void *k, const void *v, void *out, const float *S0,
             const float *z0, float *S, float *z, int B, int H, int N, int d, int dv, int chunk,
             int seg_len, int dtype, Plan *plan)
{
    if (!k || !v)
        return LA_EINVAL;
    if (form == GLOBAL) {
        if ((q == nullptr) != (out == nullptr))
            return LA_EINVAL;
    } else if (!q || !out) {
        return LA_EINVAL;
    }
    if (form == CAUSAL && ((S == nullptr) != (z == nullptr) || (S0 == nullptr) != (z0 == nullptr)))
        return LA_EINVAL;
    if (form != CAUSAL && (!S || !z || S0 || z0))
        return LA_EINVAL;
    const void *ptrs[] = {q, k, v, out, S0, z0, S, z};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return LA_EINVAL;
    const int s = make_plan(form, B, H, N, d, dv, chunk, seg_len, dtype, plan);
    if (s != LA_OK)
        return s;

    const size_t es = dtype == LA_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * (size_t)H;
    const Span sq = span(q, BH * N * d * es), sk = span(k, BH * N * d * es);
    const Span sv = span(v, BH * N * dv * es), so = span(out, BH * N * dv * es);
    const Span sS = span(S, BH * d * dv * 4), sz = span(z, BH * d * 4);
    const Span sS0 = span(S0, BH * d * dv * 4), sz0 = span(z0, BH * d * 4);
    for (Span in : {sq, sk, sv})
        if (overlap(so, in))
            return LA_EINVAL;
    for (Span st : {sS, sz, sS0, sz0})
        for (Span o : {sq, sk, sv, so})
            if (overlap(st, o))
                return LA_EINVAL;
    if (overlap(sS, sz) || overlap(sS0, sz0))
        return LA_EINVAL;
    // the initial state is either the final state's own buffers (in place) or apart from them
    if (S0 && S0 != S && (overlap(sS0, sS) || overlap(sS0, sz)))
        return LA_EINVAL;
    if (z0 && z0 != z && (overlap(sz0, sS) || overlap(sz0, sz)))
        return LA_EINVAL;
    if (S0 && ((S0 == S) != (z0 == z)))
        return LA_EINVAL;
    return LA_OK;
}

// Scratch blocks of the convenience entry points (those without a workspace argument), kept for
// the life of the process (or until la_release_cache). A call takes any free block of its
// device that is large enough and makes its stream wait, on the device, for the block's last
// use (hipStreamWaitEvent on an event recorded after that use's kernels; no wait when that use
// was on the same stream, which stream order already covers); the host never waits. When no
// free block is large enough a new one is allocated (hipMalloc). Reuse therefore depends on
// completion, not on which stream handle a block was last used with: per-thread default
// streams, streams destroyed and handles reused, and blocks of streams that no longer exist are
// all handled the same way. (Taking and returning stream-ordered pool memory in every call made
// the call wait on the host for the stream to drain, measured on MI355X: the host could not run
// ahead of the device.) HIP calls are made outside the lock.
struct BlockCache {
    struct Block {
        int dev;
        void *ptr;
        size_t bytes;
        hipEvent_t last; // recorded after the kernels of the call that last used the block
        bool used;       // `last` has been recorded at least once
        bool busy;
    };
    std::mutex mu;
    std::vector<Block *> blocks; // never shrinks except in release()

    hipError_t take(int dev, hipStream_t st, size_t bytes, Block **out)
    {
        Block *fit = nullptr;
        {
            std::lock_guard<std::mutex> lock(mu);
            for (Block *b : blocks)
                if (b->dev == dev && !b->busy && b->bytes >= bytes && (!fit || b->bytes < fit->bytes))
                    fit = b;
            if (fit)
                fit->busy = true;
        }
        if (fit) {
            const hipError_t e = fit->used ? hipStreamWaitEvent(st, fit->last, 0) : hipSuccess;
            if (e != hipSuccess) {
                std::lock_guard<std::mutex> lock(mu);
                fit->busy = false;
                return e;
            }
            *out = fit;
            return hipSuccess;
        }
        Block *b = new Block{dev, nullptr, bytes, nullptr, false, true};
        hipError_t e = hipMalloc(&b->ptr, bytes);
        if (e == hipSuccess) {
            // only kernels on this device touch the block, so the event needs no system-scope
            // fence (measured on MI355X: the fence's cache write-back cost 1.5 us per call)
            e = hipEventCreateWithFlags(&b->last, hipEventDisableTiming | hipEventDisableSystemFence);
            if (e != hipSuccess)
                (void)hipFree(b->ptr);
        }
        if (e != hipSuccess) {
            delete b;
            return e;
        }
        std::lock_guard<std::mutex> lock(mu);
        blocks.push_back(b);
        *out = b;
        return hipSuccess;
    }
    // After the call's kernels are enqueued on `st`: mark the block's last use there and free it
    // for other calls. If the mark cannot be recorded the block stays busy for good (its last
    // use would be unknown).
    hipError_t give_back(Block *b, hipStream_t st)
    {
        const hipError_t e = hipEventRecord(b->last, st);
        std::lock_guard<std::mutex> lock(mu);
        if (e == hipSuccess) {
            b->used = true;
            b->busy = false;
        }
        return e;
    }
    // Frees every block not in use by a call, after the work that last used it.
    hipError_t release()
    {
        std::vector<Block *> mine;
        {
            std::lock_guard<std::mutex> lock(mu);
            std::vector<Block *> keep;
            for (Block *b : blocks)
                (b->busy ? keep : mine).push_back(b);
            blocks.swap(keep);
        }
        hipError_t err = hipSuccess;
        for (Block *b : mine) {
            int cur = 0;
            hipError_t e = hipGetDevice(&cur);
            if (e == hipSuccess && cur != b->dev)
                e = hipSetDevice(b->dev);
            if (e == hipSuccess && b->used)
                e = hipEventSynchronize(b->last);
            if (e == hipSuccess)
                e = hipEventDestroy(b->last);
            if (e == hipSuccess)
                e = hipFree(b->ptr);
            if (cur != b->dev)
                (void)hipSetDevice(cur);
            if (e != hipSuccess) {
                err = e;
                std::lock_guard<std::mutex> lock(mu);
                blocks.push_back(b); // not freed: keep it (and its pointer) known
            } else {
                delete b;
            }
        }
        return err;
    }
};

BlockCache &block_cache()
{
    static BlockCache *c = new BlockCache(); // never destroyed: blocks live until release()
    return *c;
}

// Scratch device memory of one convenience call: a cached block (or, under stream capture,
// stream-ordered pool memory, so that every replay of the graph owns its scratch), released by
// finish() once the call's kernels are enqueued.
struct Workspace {
    float *ptr = nullptr;
    hipStream_t st = nullptr;
    BlockCache::Block *blk = nullptr;
    bool pooled = false;
    hipError_t init(size_t bytes, hipStream_t stream)
    {
        st = stream;
        if (!bytes)
            return hipSuccess;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess)
            return e;
        if (cs != hipStreamCaptureStatusNone) {
            // allocation and free nodes in the captured graph (the device's default pool:
            // measured to capture on ROCm where a private pool does not)
            e = hipMallocAsync(reinterpret_cast<void **>(&ptr), bytes, stream);
            pooled = e == hipSuccess;
            return e;
        }
        int dev = 0;
        e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        e = block_cache().take(dev, stream, bytes, &blk);
        if (e == hipSuccess)
            ptr = static_cast<float *>(blk->ptr);
        return e;
    }
    hipError_t finish()
    {
        hipError_t e = hipSuccess;
        if (pooled)
            e = hipFreeAsync(ptr, st);
        else if (blk)
            e = block_cache().give_back(blk, st);
        ptr = nullptr;
        blk = nullptr;
        pooled = false;
        return e;
    }
    ~Workspace() { (void)finish(); }
};

// Scratch of la_causal_fwd_noalloc, for callers that cannot allocate device memory: one array
// per GPU (each device holds its own copy for the life of the process), 64 MiB -- enough for
// every sequence split the library chooses for the matrix-core kernels (at most 510 segment
// states of 66,048 B at d = d_v = 128). In host code `scratch` is only a stand-in for the
// symbol: its device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed to kernels.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void **out)
{
    static std::mutex mu;
    static void *ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

// HIP events marking the phase boundaries of one causal call (profiling form only).
struct Stamps {
    hipEvent_t ev[4] = {};
    Stamps() = default;
    Stamps(const Stamps &) = delete;
    Stamps &operator=(const Stamps &) = delete;
    hipError_t init()
    {
        for (hipEvent_t &x : ev) {
            const hipError_t e = hipEventCreate(&x);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    ~Stamps()
    {
        for (hipEvent_t x : ev)
            if (x)
                (void)hipEventDestroy(x);
    }
};

hipError_t mark(Stamps *ts, int i, hipStream_t st)
{
    return ts ? hipEventRecord(ts->ev[i], st) : hipSuccess;
}

bool flags_ok(int flags) { return (flags & ~(LA_PHI_IDENTITY | LA_UNNORMALIZED)) == 0; }

// The decay vector: non-null, 4-byte aligned, H floats that no written buffer overlaps (sizes
// are checked by validate; here only what the pointer itself needs, with positive sizes).
bool gamma_ok(const float *gamma, int H, const void *out, const float *S, const float *z, int B,
              int N, int d, int dv, int dtype)
{
    if (!gamma || (reinterpret_cast<uintptr_t>(gamma) & 3u) != 0)
        return false;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || dv <= 0)
        return true; // validate reports the size error
    const size_t es = dtype == LA_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * (size_t)H;
    const Span sg = span(gamma, (size_t)H * 4);
    return !overlap(sg, span(out, BH * N * dv * es)) && !overlap(sg, span(S, BH * d * dv * 4)) &&
           !overlap(sg, span(z, BH * d * 4));
}

// gamma (optional): per-head decay of the carried state, device float32 [H]. wsp: pl.ws_bytes
// of device scratch (unused when the plan has one segment).
int run_causal(const void *q, const void *k, const void *v, void *out, const float *S0,
               const float *z0, float *S, float *z, int N, int d, int dv, bool bf16, int flags,
               const float *gamma, int H, const Plan &pl, float *wsp, hipStream_t st,
               Stamps *ts = nullptr)
{
    const int BH = (int)pl.BH, P = pl.P, L = pl.L;
    const long E = (long)d * dv + d;
    hipError_t e = mark(ts, 0, st);
    const float *preS = S0, *prez = z0; // P == 1: the initial state (or none) is the prefix
    long ps = (long)d * dv, pzs = d;
    int pm = 0;
    if (P > 1 && e == hipSuccess && pl.mfma) {
        // sums of segments 0..P-2, with the initial state copied into slot P-1; each causal
        // segment then adds up the sums before it (no scan launch)
        e = la::agg_mfma(d, flags, k, v, wsp, wsp + (long)d * dv, E, E, BH, N, L, P - 1, P, gamma,
                         H, S0, z0, st);
        if (e == hipSuccess)
            e = mark(ts, 1, st);
        pm = la::PM_SUMS | (S0 ? la::PM_INIT : 0) | (BH % 8 == 0 ? la::PM_XCD : 0);
        preS = wsp;
        prez = wsp + (long)d * dv;
        ps = pzs = E;
    } else if (P > 1 && e == hipSuccess) {
        // sums of segments 0..P-2, then the exclusive prefix over segments in place
        e = pl.mfma32 ? la::agg_mfma32(d, flags, k, v, wsp, wsp + (long)d * dv, E, E, BH, N, L,
                                       P - 1, P, gamma, H, st)
                      : la::agg_valu(bf16, flags, k, v, wsp, wsp + (long)d * dv, E, E, BH, N,
                                     d, dv, pl.chunk, L, P - 1, P, gamma, H, st);
        if (e == hipSuccess)
            e = mark(ts, 1, st);
        if (e == hipSuccess)
            e = la::seg_exclusive_scan(wsp, S0, z0, BH, P, d, dv, gamma, H, L, st);
        preS = wsp;
        prez = wsp + (long)d * dv;
        ps = pzs = E;
    } else if (e == hipSuccess) {
        e = mark(ts, 1, st);
    }
    if (e == hipSuccess)
        e = mark(ts, 2, st);
    if (e == hipSuccess)
        e = pl.mfma ? la::causal_mfma(d, flags, q, k, v, out, preS, prez, ps, pzs, pm, S, z, BH, N,
                                      L, P, gamma, H, st)
            : pl.mfma32 ? la::causal_mfma32(d, flags, q, k, v, out, preS, prez, ps, pzs, S, z, BH, N,
                                        L, P, gamma, H, st)
            : pl.shortseq && !gamma
                ? la::short_causal(bf16, flags, q, k, v, out, S0, z0, S, z, BH, N, d, dv, st)
                : la::out_valu(bf16, true, flags, q, k, v, out, preS, prez, ps, pzs, P > 1 ? P : 1, S,
                               z, BH, N, d, dv, pl.chunk, L, P, gamma, H, st);
    if (e == hipSuccess)
        e = mark(ts, 3, st);
    return e == hipSuccess ? LA_OK : LA_EHIP;
}

int run_global(const void *q, const void *k, const void *v, void *out, float *S, float *z, int N,
               int d, int dv, bool bf16, int flags, const Plan &pl, float *wsp, hipStream_t st)
{
    const int BH = (int)pl.BH, P = pl.P, L = pl.L;
    const long E = (long)d * dv + d;
    hipError_t e;
    if (P > 1) {
        e = pl.mfma   ? la::agg_mfma(d, flags, k, v, wsp, wsp + (long)d * dv, E, E, BH, N, L,
                                     P, P, nullptr, 1, nullptr, nullptr, st)
            : pl.mfma32 ? la::agg_mfma32(d, flags, k, v, wsp, wsp + (long)d * dv, E, E, BH, N,
                                         L, P, P, nullptr, 1, st)
                      : la::agg_valu(bf16, flags, k, v, wsp, wsp + (long)d * dv, E, E, BH, N,
                                     d, dv, pl.chunk, L, P, P, nullptr, 1, st);
        if (e == hipSuccess)
            e = la::seg_total(wsp, S, z, BH, P, d, dv, st);
    } else {
        e = pl.mfma   ? la::agg_mfma(d, flags, k, v, S, z, (long)d * dv, d, BH, N, L, 1, 1,
                                     nullptr, 1, nullptr, nullptr, st)
            : pl.mfma32 ? la::agg_mfma32(d, flags, k, v, S, z, (long)d * dv, d, BH, N, L, 1, 1,
                                         nullptr, 1, st)
                      : la::agg_valu(bf16, flags, k, v, S, z, (long)d * dv, d, BH, N, d, dv,
                                     pl.chunk, L, 1, 1, nullptr, 1, st);
    }
    if (e == hipSuccess && q)
        e = pl.mfma   ? la::global_read_mfma(d, flags, q, out, S, z, BH, N, L, P, st)
            : pl.mfma32 ? la::global_read_mfma32(d, flags, q, out, S, z, BH, N, st)
                      : la::out_valu(bf16, false, flags, q, nullptr, nullptr, out, S, z, (long)d * dv,
                                   d, 1, nullptr, nullptr, BH, N, d, dv, pl.chunk, L, P, nullptr, 1,
                                   st);
    return e == hipSuccess ? LA_OK : LA_EHIP;
}

// The convenience forms: scratch from the library's cache (or the stream-ordered pool under
// capture), released once the call's kernels are enqueued.
int run_causal_cached(const void *q, const void *k, const void *v, void *out, const float *S0,
                      const float *z0, float *S, float *z, int N, int d, int dv, bool bf16,
                      int flags, const float *gamma, int H, const Plan &pl, hipStream_t st,
                      Stamps *ts = nullptr)
{
    Workspace ws;
    if (ws.init(pl.ws_bytes, st) != hipSuccess)
        return LA_EHIP;
    const int r = run_causal(q, k, v, out, S0, z0, S, z, N, d, dv, bf16, flags, gamma, H, pl, ws.ptr,
                             st, ts);
    const hipError_t e = ws.finish();
    return r != LA_OK ? r : (e == hipSuccess ? LA_OK : LA_EHIP);
}

int run_global_cached(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                      int N, int d, int dv, bool bf16, int flags, const Plan &pl, hipStream_t st)
{
    Workspace ws;
    if (ws.init(pl.ws_bytes, st) != hipSuccess)
        return LA_EHIP;
    const int r = run_global(q, k, v, out, S, z, N, d, dv, bf16, flags, pl, ws.ptr, st);
    const hipError_t e = ws.finish();
    return r != LA_OK ? r : (e == hipSuccess ? LA_OK : LA_EHIP);
}

// A caller-supplied workspace: large enough for the plan, 16-byte aligned (or NULL when the plan
// needs none), and apart from every buffer the call reads or writes.
bool workspace_ok(const void *ws, size_t ws_bytes, const Plan &pl, const std::vector<Span> &bufs)
{
    if (!pl.ws_bytes)
        return true;
    if (!ws || !aligned16(ws) || ws_bytes < pl.ws_bytes)
        return false;
    const Span w = span(ws, pl.ws_bytes);
    for (Span b : bufs)
        if (overlap(w, b))
            return false;
    return true;
}

// The buffers of a causal or global call, as validate() sized them.
std::vector<Span> call_spans(const void *q, const void *k, const void *v, const void *out,
                             const float *S0, const float *z0, const float *S, const float *z,
                             const float *gamma, int B, int H, int N, int d, int dv, int dtype)
{
    const size_t es = dtype == LA_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * (size_t)H;
    return {span(q, BH * N * d * es),   span(k, BH * N * d * es),   span(v, BH * N * dv * es),
            span(out, BH * N * dv * es), span(S0, BH * d * dv * 4), span(z0, BH * d * 4),
            span(S, BH * d * dv * 4),   span(z, BH * d * 4),        span(gamma, (size_t)H * 4)};
}

// The random-feature causal call: q, k [B,H,N,d] are mapped with W [m, d] to features
// [B,H,N,m] and the causal identity-map form runs over them (S [B,H,m,d_v], z [B,H,m]). When
// m == d == d_v in {64, 128} and the matrix-core kernels apply, the map runs inside their
// staging (no feature tensor is written); otherwise the features go through scratch memory.
int validate_rf(const void *q, const void *k, const void *v, void *out, const void *W,
                const float *S0, const float *z0, float *S, float *z, int B, int H, int N, int d,
                int dv, int m, int chunk, int seg_len, int flags, int dtype, Plan *plan)
{
    if (!flags_ok(flags) || (flags & LA_PHI_IDENTITY))
        return LA_EINVAL;
    if (!q || !k || !v || !out || !W)
        return LA_EINVAL;
    if ((S == nullptr) != (z == nullptr) || (S0 == nullptr) != (z0 == nullptr))
        return LA_EINVAL;
    const void *ptrs[] = {q, k, v, out, W, S0, z0, S, z};
    for (const void *p : ptrs)
        if (p && !aligned16(p))
            return LA_EINVAL;
    if (dtype != LA_F32 && dtype != LA_BF16)
        return LA_EINVAL;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || dv <= 0 || m <= 0 || chunk < 0 || seg_len < 0)
        return LA_EINVAL;
    if (d > la::rf_max_d())
        return LA_ENOTSUP;
    // the attention runs over m features
    const int s = make_plan(CAUSAL, B, H, N, m, dv, chunk, seg_len, dtype, plan);
    if (s != LA_OK)
        return s;
    if ((size_t)N * (size_t)d > (size_t)INT32_MAX || (size_t)B * H * N > (size_t)INT32_MAX)
        return LA_ENOTSUP;
    const size_t es = dtype == LA_BF16 ? 2 : 4;
    const size_t BH = (size_t)B * (size_t)H;
    const Span sq = span(q, BH * N * d * es), sk = span(k, BH * N * d * es);
    const Span sv = span(v, BH * N * dv * es), so = span(out, BH * N * dv * es);
    const Span sw = span(W, (size_t)m * d * es);
    const Span sS = span(S, BH * m * dv * 4), sz = span(z, BH * m * 4);
    const Span sS0 = span(S0, BH * m * dv * 4), sz0 = span(z0, BH * m * 4);
    for (Span in : {sq, sk, sv, sw})
        if (overlap(so, in))
            return LA_EINVAL;
    for (Span st : {sS, sz, sS0, sz0})
        for (Span o : {sq, sk, sv, so, sw})
            if (overlap(st, o))
                return LA_EINVAL;
    if (overlap(sS, sz) || overlap(sS0, sz0))
        return LA_EINVAL;
    if (S0 && S0 != S && (overlap(sS0, sS) || overlap(sS0, sz)))
        return LA_EINVAL;
    if (z0 && z0 != z && (overlap(sz0, sS) || overlap(sz0, sz)))
        return LA_EINVAL;
    if (S0 && ((S0 == S) != (z0 == z)))
        return LA_EINVAL;
    return LA_OK;
}

int run_causal_rf(const void *q, const void *k, const void *v, void *out, const void *W,
                  const float *S0, const float *z0, float *S, float *z, int N, int d, int dv,
                  int m, bool bf16, int flags, const Plan &pl, hipStream_t st)
{
    const int BH = (int)pl.BH, P = pl.P, L = pl.L;
    if (pl.mfma && m == d && d == dv) {
        const long E = (long)d * dv + d;
        Workspace ws;
        if (ws.init(pl.ws_bytes, st) != hipSuccess)
            return LA_EHIP;
        hipError_t e = hipSuccess;
        const float *preS = S0, *prez = z0;
        long ps = (long)d * dv, pzs = d;
        int pm = 0;
        if (P > 1) {
            // as in the plain form: the sums and the initial state in the workspace, each
            // causal segment adds up the sums before it
            e = la::agg_rf_mfma(d, k, v, W, ws.ptr, ws.ptr + (long)d * dv, E, E, BH, N, L, P - 1, P,
                                S0, z0, st);
            pm = la::PM_SUMS | (S0 ? la::PM_INIT : 0) | (BH % 8 == 0 ? la::PM_XCD : 0);
            preS = ws.ptr;
            prez = ws.ptr + (long)d * dv;
            ps = pzs = E;
        }
        if (e == hipSuccess)
            e = la::causal_rf_mfma(d, flags, q, k, v, W, out, preS, prez, ps, pzs, pm, S, z, BH, N, L,
                                   P, st);
        const hipError_t ef = ws.finish();
        return e == hipSuccess && ef == hipSuccess ? LA_OK : LA_EHIP;
    }
    // features through scratch memory, then the identity-map causal form over them
    const size_t es = bf16 ? 2 : 4;
    const size_t fbytes = (size_t)BH * N * m * es;
    Workspace feat;
    if (feat.init(2 * fbytes, st) != hipSuccess)
        return LA_EHIP;
    char *fq = reinterpret_cast<char *>(feat.ptr), *fk = fq + fbytes;
    const long rows = (long)BH * N;
    hipError_t e = la::rf_features(bf16, q, W, fq, rows, d, m, st);
    if (e == hipSuccess)
        e = la::rf_features(bf16, k, W, fk, rows, d, m, st);
    if (e != hipSuccess)
        return LA_EHIP;
    const int r = run_causal_cached(fq, fk, v, out, S0, z0, S, z, N, m, dv, bf16,
                                    flags | LA_PHI_IDENTITY, nullptr, 1, pl, st);
    const hipError_t ef = feat.finish();
    return r != LA_OK ? r : (ef == hipSuccess ? LA_OK : LA_EHIP);
}

} // namespace

extern "C" {

int la_causal_fwd_ex(const void *q, const void *k, const void *v, void *out, const float *S0,
                     const float *z0, float *S, float *z, int B, int H, int N, int d, int d_v,
                     int chunk, int seg_len, int flags, la_dtype dtype, hipStream_t stream)
{
    if (!flags_ok(flags))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(CAUSAL, q, k, v, out, S0, z0, S, z, B, H, N, d, d_v, chunk, seg_len,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    return run_causal_cached(q, k, v, out, S0, z0, S, z, N, d, d_v, dtype == LA_BF16, flags, nullptr,
                             1, pl, stream);
}

int la_causal_fwd_decay(const void *q, const void *k, const void *v, void *out, const float *S0,
                        const float *z0, float *S, float *z, const float *gamma, int B, int H,
                        int N, int d, int d_v, int chunk, int seg_len, int flags, la_dtype dtype,
                        hipStream_t stream)
{
    if (!flags_ok(flags) || !gamma_ok(gamma, H, out, S, z, B, N, d, d_v, dtype))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(CAUSAL, q, k, v, out, S0, z0, S, z, B, H, N, d, d_v, chunk, seg_len,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    return run_causal_cached(q, k, v, out, S0, z0, S, z, N, d, d_v, dtype == LA_BF16, flags, gamma,
                             H, pl, stream);
}

int la_causal_fwd_state(const void *q, const void *k, const void *v, void *out, const float *S0,
                        const float *z0, float *S, float *z, int B, int H, int N, int d, int d_v,
                        int chunk, int seg_len, la_dtype dtype, hipStream_t stream)
{
    return la_causal_fwd_ex(q, k, v, out, S0, z0, S, z, B, H, N, d, d_v, chunk, seg_len, 0, dtype,
                            stream);
}
int la_causal_fwd_seg(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                      int B, int H, int N, int d, int d_v, int chunk, int seg_len, la_dtype dtype,
                      hipStream_t stream)
{
    return la_causal_fwd_state(q, k, v, out, S, z, S, z, B, H, N, d, d_v, chunk, seg_len, dtype,
                               stream);
}

int la_causal_fwd_profiled(const void *q, const void *k, const void *v, void *out,
                           const float *S0, const float *z0, float *S, float *z, int B, int H,
                           int N, int d, int d_v, int chunk, int seg_len, int flags, la_dtype dtype,
                           hipStream_t stream, int reps, float *ms)
{
    if (!ms || reps < 1 || reps > 4096 || !flags_ok(flags))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(CAUSAL, q, k, v, out, S0, z0, S, z, B, H, N, d, d_v, chunk, seg_len,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    std::vector<Stamps> ts(reps);
    for (Stamps &t : ts)
        if (t.init() != hipSuccess)
            return LA_EHIP;
    for (Stamps &t : ts) {
        const int r = run_causal_cached(q, k, v, out, S0, z0, S, z, N, d, d_v, dtype == LA_BF16,
                                        flags, nullptr, 1, pl, stream, &t);
        if (r != LA_OK)
            return r;
    }
    if (hipEventSynchronize(ts.back().ev[3]) != hipSuccess)
        return LA_EHIP;
    double sum[3] = {0.0, 0.0, 0.0};
    for (Stamps &t : ts)
        for (int i = 0; i < 3; ++i) {
            float x = 0.f;
            if (hipEventElapsedTime(&x, t.ev[i], t.ev[i + 1]) != hipSuccess)
                return LA_EHIP;
            sum[i] += x;
        }
    for (int i = 0; i < 3; ++i)
        ms[i] = (float)(sum[i] / reps);
    return LA_OK;
}

int la_causal_fwd(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                  int B, int H, int N, int d, int d_v, int chunk, la_dtype dtype, hipStream_t stream)
{
    return la_causal_fwd_seg(q, k, v, out, S, z, B, H, N, d, d_v, chunk, 0, dtype, stream);
}

int la_global_fwd_ex(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                     int B, int H, int N, int d, int d_v, int chunk, int flags, la_dtype dtype,
                     hipStream_t stream)
{
    if (!flags_ok(flags))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(GLOBAL, q, k, v, out, nullptr, nullptr, S, z, B, H, N, d, d_v, chunk, 0,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    return run_global_cached(q, k, v, out, S, z, N, d, d_v, dtype == LA_BF16, flags, pl, stream);
}

int la_causal_fwd_ws(const void *q, const void *k, const void *v, void *out, const float *S0,
                     const float *z0, float *S, float *z, const float *gamma, int B, int H, int N,
                     int d, int d_v, int chunk, int seg_len, int flags, la_dtype dtype, void *ws,
                     size_t ws_bytes, hipStream_t stream)
{
    if (!flags_ok(flags) || (gamma && !gamma_ok(gamma, H, out, S, z, B, N, d, d_v, dtype)))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(CAUSAL, q, k, v, out, S0, z0, S, z, B, H, N, d, d_v, chunk, seg_len,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    if (!workspace_ok(ws, ws_bytes, pl,
                      call_spans(q, k, v, out, S0, z0, S, z, gamma, B, H, N, d, d_v, dtype)))
        return LA_EINVAL;
    return run_causal(q, k, v, out, S0, z0, S, z, N, d, d_v, dtype == LA_BF16, flags, gamma,
                      gamma ? H : 1, pl, static_cast<float *>(ws), stream);
}

int la_global_fwd_ws(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                     int B, int H, int N, int d, int d_v, int chunk, int flags, la_dtype dtype,
                     void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!flags_ok(flags))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(GLOBAL, q, k, v, out, nullptr, nullptr, S, z, B, H, N, d, d_v, chunk, 0,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    if (!workspace_ok(ws, ws_bytes, pl,
                      call_spans(q, k, v, out, nullptr, nullptr, S, z, nullptr, B, H, N, d, d_v,
                                 dtype)))
        return LA_EINVAL;
    return run_global(q, k, v, out, S, z, N, d, d_v, dtype == LA_BF16, flags, pl,
                      static_cast<float *>(ws), stream);
}

int la_causal_fwd_noalloc(const void *q, const void *k, const void *v, void *out,
                          const float *S0, const float *z0, float *S, float *z, int B, int H,
                          int N, int d, int d_v, int chunk, int seg_len, int flags, la_dtype dtype,
                          hipStream_t stream)
{
    if (!flags_ok(flags))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(CAUSAL, q, k, v, out, S0, z0, S, z, B, H, N, d, d_v, chunk, seg_len,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    if (pl.ws_bytes > kStaticScratchBytes)
        return LA_ENOSPACE;
    void *ws = nullptr;
    if (pl.ws_bytes && static_scratch(&ws) != hipSuccess)
        return LA_EHIP;
    return run_causal(q, k, v, out, S0, z0, S, z, N, d, d_v, dtype == LA_BF16, flags, nullptr, 1, pl,
                      static_cast<float *>(ws), stream);
}

int la_release_cache(void)
{
    return block_cache().release() == hipSuccess ? LA_OK : LA_EHIP;
}

int la_global_fwd(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                  int B, int H, int N, int d, int d_v, int chunk, la_dtype dtype, hipStream_t stream)
{
    return la_global_fwd_ex(q, k, v, out, S, z, B, H, N, d, d_v, chunk, 0, dtype, stream);
}

int la_decode_step_ex(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                      int B, int H, int N, int d, int d_v, int flags, la_dtype dtype,
                      hipStream_t stream)
{
    if (!flags_ok(flags))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(DECODE, q, k, v, out, nullptr, nullptr, S, z, B, H, N, d, d_v, 0, 0,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    const hipError_t e = la::decode_step(dtype == LA_BF16, flags, q, k, v, out, S, z, (int)pl.BH,
                                         d, d_v, nullptr, 1, stream);
    return e == hipSuccess ? LA_OK : LA_EHIP;
}

int la_decode_step_decay(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                         const float *gamma, int B, int H, int N, int d, int d_v, int flags,
                         la_dtype dtype, hipStream_t stream)
{
    if (!flags_ok(flags) || !gamma_ok(gamma, H, out, S, z, B, N, d, d_v, dtype))
        return LA_EINVAL;
    Plan pl;
    const int s = validate(DECODE, q, k, v, out, nullptr, nullptr, S, z, B, H, N, d, d_v, 0, 0,
                           dtype, &pl);
    if (s != LA_OK)
        return s;
    const hipError_t e = la::decode_step(dtype == LA_BF16, flags, q, k, v, out, S, z, (int)pl.BH,
                                         d, d_v, gamma, H, stream);
    return e == hipSuccess ? LA_OK : LA_EHIP;
}

int la_decode_step(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                   int B, int H, int N, int d, int d_v, int chunk, la_dtype dtype,
                   hipStream_t stream)
{
    (void)chunk;
    return la_decode_step_ex(q, k, v, out, S, z, B, H, N, d, d_v, 0, dtype, stream);
}

int la_causal_fwd_rf(const void *q, const void *k, const void *v, void *out, const void *W,
                     const float *S0, const float *z0, float *S, float *z, int B, int H, int N,
                     int d, int d_v, int m, int chunk, int seg_len, int flags, la_dtype dtype,
                     hipStream_t stream)
{
    Plan pl;
    const int s = validate_rf(q, k, v, out, W, S0, z0, S, z, B, H, N, d, d_v, m, chunk, seg_len,
                              flags, dtype, &pl);
    if (s != LA_OK)
        return s;
    return run_causal_rf(q, k, v, out, W, S0, z0, S, z, N, d, d_v, m, dtype == LA_BF16, flags, pl,
                         stream);
}

int la_rf_features(const void *x, const void *W, void *f, long rows, int d, int m,
                   la_dtype dtype, hipStream_t stream)
{
    if (!x || !W || !f || !aligned16(x) || !aligned16(W) || !aligned16(f))
        return LA_EINVAL;
    if (dtype != LA_F32 && dtype != LA_BF16)
        return LA_EINVAL;
    if (rows <= 0 || d <= 0 || m <= 0)
        return LA_EINVAL;
    if (d > la::rf_max_d() || m > kRfMaxFeatures || rows > (long)INT32_MAX)
        return LA_ENOTSUP;
    const size_t es = dtype == LA_BF16 ? 2 : 4;
    const Span sf = span(f, (size_t)rows * m * es);
    if (overlap(sf, span(x, (size_t)rows * d * es)) || overlap(sf, span(W, (size_t)m * d * es)))
        return LA_EINVAL;
    const hipError_t e = la::rf_features(dtype == LA_BF16, x, W, f, rows, d, m, stream);
    return e == hipSuccess ? LA_OK : LA_EHIP;
}

size_t la_workspace_bytes(int form, int B, int H, int N, int d, int d_v, int chunk, int seg_len,
                          la_dtype dtype)
{
    if (form != 0 && form != 1)
        return 0;
    Plan pl;
    if (make_plan(form == 0 ? CAUSAL : GLOBAL, B, H, N, d, d_v, chunk, seg_len, dtype, &pl) != LA_OK)
        return 0;
    return pl.ws_bytes;
}

int la_segments(int form, int B, int H, int N, int d, int d_v, int chunk, int seg_len,
                la_dtype dtype)
{
    if (form != 0 && form != 1)
        return 0;
    Plan pl;
    if (make_plan(form == 0 ? CAUSAL : GLOBAL, B, H, N, d, d_v, chunk, seg_len, dtype, &pl) != LA_OK)
        return 0;
    return pl.P;
}

const char *la_strerror(int status)
{
    switch (status) {
    case LA_OK:
        return "success";
    case LA_EINVAL:
        return "invalid argument (null, misaligned or overlapping buffer, non-positive size, "
               "decode with N != 1, unknown dtype or unknown flag bits)";
    case LA_ENOTSUP:
        return "unsupported shape or chunk (d and d_v must be 16, 32, 64 or 128; chunk 0, 16, "
               "32, 64 or 128 as the shape allows; random features: d <= 256, m <= 4096)";
    case LA_EHIP:
        return "HIP runtime error (allocation or kernel launch failed)";
    case LA_ENOSPACE:
        return "the call needs more scratch than the library's static scratch array holds "
               "(64 MiB per device; la_causal_fwd_noalloc)";
    default:
        return "unknown status";
    }
}

int la_version(void) { return LA_VERSION; }

} // extern "C"
